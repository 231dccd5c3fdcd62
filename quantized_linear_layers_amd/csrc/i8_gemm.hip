// W8A8 GEMM: int8 x int8 -> int32 on v_mfma_i32_32x32x32_i8, with the scale
// and zero-point epilogue applied to the accumulators in registers before
// the single store of the output ([VE] "一、背景": fusing it into the GEMM's
// epilogue avoids writing and re-reading the int32 result; [VE] "2.4": the
// per-token zero point is a rank-1 correction azp[m] * azp_adj[n], applied
// element-wise with O(M + N) extra memory).
//
// Each workgroup (4 waves, 2 x 2 waves of 64 x 64) owns a 128 x 128 tile and
// walks K in blocks of 64 bytes through a ring of kStages LDS slots (64 KB, so
// that two workgroups share a compute unit and hide each other's waits).  The
// slots are filled straight from global memory by global_load_lds_dwordx4
// (no register staging), kStages - 1 blocks ahead of the block being
// multiplied, so the L2 / Infinity-cache latency of an operand block is
// hidden behind the MFMAs of the blocks before it.  Each slot is its own LDS
// object and the K loop is unrolled by kStages, so every LDS read names the
// slot it depends on and waits only for that slot's loads.  Rows of a slot
// are 64 bytes (4 pieces of 16 bytes) stored with the piece index XORed by
// row bits, so the rows one MFMA operand read touches spread over the banks.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;       // BK in bytes (int8 elements)
constexpr int kStages = 4;
constexpr int kSlot = BM * BK;                   // bytes of one operand tile (A and B are the same size)
constexpr int kPieces = BK / 16;                 // 16-byte pieces per row

// one LDS object per stage holding the A tile then the B tile
__shared__ __align__(1024) int8_t st0[2 * kSlot], st1[2 * kSlot], st2[2 * kSlot], st3[2 * kSlot];

template <int S>
__device__ inline int8_t* slot_a() {
  if constexpr (S == 0) return st0; else if constexpr (S == 1) return st1; else if constexpr (S == 2) return st2;
  else return st3;
}
template <int S>
__device__ inline int8_t* slot_b() { return slot_a<S>() + kSlot; }

struct I8Args {
  const int8_t* A;
  const int8_t* B;
  int M, N, K;
  I8Epi e;
};

// byte offset of logical 16-byte piece p of row r inside a slot: the piece
// index is XORed with bits 1..2 of the row, so 8 consecutive rows read at one
// logical piece touch 8 different 16-byte bank groups
__device__ inline int swz(int r, int p) { return r * BK + ((p ^ ((r >> 1) & 3)) << 4); }

// issues one 16-byte global -> LDS load per lane (lane i writes lds + 16 i)
__device__ inline void load_lds16(const int8_t* src, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), lds, 16, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

// One wave's share of filling a slot: the slot holds 8 blocks of 1 KB
// (16 rows x 64 bytes) per operand, kFills = 2 per wave.  Lane l of a block
// writes LDS bytes 16 l .. 16 l + 15 of the block, i.e. row l / 4 and stored
// piece l % 4, which holds logical piece (l % 4) ^ ((row >> 1) & 3).  Rows
// past M or N are clamped to the last row (valid loads whose data only
// reaches outputs that are never stored).
constexpr int kFills = kSlot / 1024 / 4;         // 1 KB blocks per operand per wave and slot fill

struct FillPlan {
  const int8_t* a[kFills];
  const int8_t* b[kFills];
  int p16[kFills];     // byte offset of this lane's logical piece inside a K block
  int dst[kFills];     // byte offset of the lane's 1 KB destination block inside a slot
};

__device__ inline FillPlan make_fill_plan(const I8Args& a, int m0, int n0, int wave, int lane) {
  FillPlan f;
#pragma unroll
  for (int i = 0; i < kFills; ++i) {
    const int blkid = wave * kFills + i;           // 1 KB block of the slot
    const int r = blkid * (1024 / BK) + lane / kPieces;
    const int m = min(m0 + r, a.M - 1), n = min(n0 + r, a.N - 1);
    f.a[i] = a.A + (size_t)m * a.K;
    f.b[i] = a.B + (size_t)n * a.K;
    f.p16[i] = ((lane % kPieces) ^ ((r >> 1) & 3)) * 16;
    f.dst[i] = blkid * 1024;
  }
  return f;
}

// K offsets past the end of a row are clamped to the row's last 16 bytes
// (their data is zeroed before use: see mma_block)
template <int S>
__device__ inline void fill(const FillPlan& f, int kb, int K) {
#pragma unroll
  for (int i = 0; i < kFills; ++i) {
    const int k = min(kb * BK + f.p16[i], K - 16);
    load_lds16(f.a[i] + k, slot_a<S>() + f.dst[i]);
    load_lds16(f.b[i] + k, slot_b<S>() + f.dst[i]);
  }
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
// read, and lds_wait below before the fragments are used.
__device__ inline i32x4 lds_read16(const int8_t* p) {
  typedef __attribute__((address_space(3))) const int8_t* lds_ptr;
  const uint32_t off = (uint32_t)(uintptr_t)(lds_ptr)p;      // byte offset inside LDS
  i32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(off) : "memory");
#else
  v = i32x4{(int)off, 0, 0, 0};   // host pass only (never executed)
#endif
  return v;
}
// waits for this wave's LDS reads and makes the fragments depend on the wait
__device__ inline void lds_wait(i32x4& a0, i32x4& a1, i32x4& b0, i32x4& b1) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1) : : "memory");
#endif
}

// kvalid: bytes of this K block inside the matrix (BK except in a ragged last
// block); pieces past it hold whatever the clamped loads fetched and are zeroed
// here.  Rows past M or N need no masking: they only reach outputs that are
// never stored.
template <int S>
__device__ inline void mma_block(i32x16 (&acc)[2][2], int wm, int wn, int lane, int kvalid) {
  const int8_t* sa = slot_a<S>();
  const int8_t* sb = slot_b<S>();
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < BK / 32; ++ks) {
    // operand layout of the 32x32x32 int8 MFMA: lane l supplies row/column l%32,
    // bytes 16 * (l / 32) .. +16 of the 32-byte k step
    const int p = ks * 2 + half;
    i32x4 af[2], bf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      af[t] = lds_read16(sa + swz(wm + t * 32 + l32, p));
      bf[t] = lds_read16(sb + swz(wn + t * 32 + l32, p));
    }
    lds_wait(af[0], af[1], bf[0], bf[1]);
    const bool live = p * 16 < kvalid;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      af[t] = live ? af[t] : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
  }
}

// one k-block: wait for slot S, barrier, refill the slot freed by the previous
// block with block kb + kStages - 1 (clamped to the last block near the end, so
// that every wave always has the same number of loads in flight), multiply slot S
template <int S>
__device__ inline void kstep(const I8Args& a, const FillPlan& f, i32x16 (&acc)[2][2], int kb, int nkb, int wm, int wn,
                             int lane) {
  // this wave's loads of block kb are done once at most (kStages - 2) blocks
  // of its loads (2 * kFills each) remain in flight
  wait_vm<(kStages - 2) * 2 * kFills>();
  __builtin_amdgcn_s_barrier();                  // every wave's loads of block kb landed,
                                                 // and every wave finished block kb - 1
  constexpr int F = (S + kStages - 1) % kStages;
  fill<F>(f, min(kb + kStages - 1, nkb - 1), a.K);
  mma_block<S>(acc, wm, wn, lane, a.K - kb * BK);
}

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs, each
// with its own L2; when the tile count allows, consecutive tiles of a grouped
// order (8 tile rows at a time) go to one XCD, so an XCD works on an 8 x 8
// block of tiles and its L2 serves the A and B rows those tiles share.
__device__ inline void tile_of(int bid, int tm, int tn, int& mt, int& nt) {
  const int T = tm * tn;
  const int t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  constexpr int GM = 8;
  const int gsize = GM * tn;
  const int first = (t / gsize) * GM;
  const int gm = min(tm - first, GM);
  mt = first + (t % gsize) % gm;
  nt = (t % gsize) / gm;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void i8_gemm_kernel(I8Args a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int mt, nt;
  tile_of(blockIdx.x, (a.M + BM - 1) / BM, (a.N + BN - 1) / BN, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nkb = (a.K + BK - 1) / BK;

  i32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // prologue: blocks 0 .. kStages - 2 in flight (clamped to the last block)
  const FillPlan f = make_fill_plan(a, m0, n0, wave, lane);
  fill<0>(f, 0, a.K);
  fill<1>(f, min(1, nkb - 1), a.K);
  fill<2>(f, min(2, nkb - 1), a.K);

  int kb = 0;
  for (; kb + kStages <= nkb; kb += kStages) {
    kstep<0>(a, f, acc, kb, nkb, wm, wn, lane);
    kstep<1>(a, f, acc, kb + 1, nkb, wm, wn, lane);
    kstep<2>(a, f, acc, kb + 2, nkb, wm, wn, lane);
    kstep<3>(a, f, acc, kb + 3, nkb, wm, wn, lane);
  }
  if (kb < nkb) {
    kstep<0>(a, f, acc, kb, nkb, wm, wn, lane);
    if (kb + 1 < nkb) {
      kstep<1>(a, f, acc, kb + 1, nkb, wm, wn, lane);
      if (kb + 2 < nkb) kstep<2>(a, f, acc, kb + 2, nkb, wm, wn, lane);
    }
  }
  wait_vm<0>();                                  // no load may still target LDS at exit

  // ---- fused epilogue: C = Dq - azp*azp_adj (int32), out = s_a * (s_b * C) + bias.
  // Every per-row and per-column parameter is read before the first store
  // (a load after a store the compiler cannot prove disjoint would wait for a
  // full memory round trip per element): the tile's 128 row scales and zero
  // points go through LDS (the operand slots are free now), the two columns of
  // a lane through registers.
  const I8Epi& e = a.e;
  float* row_s = reinterpret_cast<float*>(st0);
  int32_t* row_z = reinterpret_cast<int32_t*>(st0 + BM * 4);
  __syncthreads();                               // every wave is done with the slots
  if (tid < BM) {
    const int m = min(m0 + tid, a.M - 1);
    row_s[tid] = e.s_a[e.s_a_vec ? m : 0];
    row_z[tid] = e.azp ? e.azp[m] : 0;
  }
  const int half = lane >> 5, l32 = lane & 31;
  float col_s[2], col_b[2];
  int32_t col_adj[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = min(n0 + wn + nt * 32 + l32, a.N - 1);
    col_s[nt] = e.s_b[e.s_b_vec ? n : 0];
    col_adj[nt] = e.azp_adj ? e.azp_adj[n] : 0;
    float b = 0.0f;
    if (e.bias) {
      const uint16_t bb = static_cast<const uint16_t*>(e.bias)[n];
      b = OUT_BF16 ? __builtin_bit_cast(float, (uint32_t)bb << 16) : (float)__builtin_bit_cast(_Float16, bb);
    }
    col_b[nt] = b;
  }
  __syncthreads();
  const bool per_token_azp = e.azp != nullptr;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + wn + nt * 32 + l32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        // acc element el of lane l: row 8*(el/4) + 4*(l/32) + el%4, column l%32
        const int r = wm + mt * 32 + 8 * (el >> 2) + 4 * half + (el & 3);
        const int m = m0 + r;
        if (m >= a.M || n >= a.N) continue;
        const int32_t c = acc[mt][nt][el] - (per_token_azp ? row_z[r] * col_adj[nt] : col_adj[nt]);
        if (e.raw) e.raw[(size_t)m * a.N + n] = c;
        const float v = row_s[r] * (col_s[nt] * (float)c) + col_b[nt];
        static_cast<uint16_t*>(e.out)[(size_t)m * a.N + n] =
            OUT_BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

}  // namespace

hipError_t launch_i8_gemm(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  I8Args a{A, B, M, N, K, e};
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (e.out_bf16)
    hipLaunchKernelGGL(i8_gemm_kernel<true>, dim3(tiles), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(i8_gemm_kernel<false>, dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ql
