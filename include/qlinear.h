/*
 * qlinear.h — C ABI of the MI355X (gfx950) quantized linear layer library
 * (libqlinear.so).
 *
 * The layer is Y = X · Wᵀ with dequantization fused into the matrix product,
 * in two modes:
 *
 *   W4A16  packed uint4 weights with one fp16 scale and one uint4 zero point
 *          per group of 128 input channels; 16-bit activations; fp32
 *          accumulation; x_fp ≈ s · (x_int − z).
 *   W8A8   int8 × int8 products accumulated in int32, then a fused epilogue
 *          out = s_a · s_b · (Dq − azp · azp_adj) + bias before the single store;
 *          or FP8 (E4M3) × FP8 products accumulated in fp32 with the scales
 *          applied in the same epilogue.
 *
 * Sources (page title, then the page's own section heading):
 *   [QK] "第 9 章 量化 Kernel：INT8 / FP8 / INT4" (Quantization kernels:
 *        INT8 / FP8 / INT4), yangyitao.com CUDA book, chapter 9.
 *   [LQ] "LLM 与 AIGC 量化：从数值格式到 W4A4" (LLM and AIGC quantization:
 *        from number formats to W4A4), valdrada.cn.
 *   [VE] "vLLM W8A8 量化 GEMM 的 CUTLASS Epilogue 设计" (the CUTLASS
 *        epilogue design of vLLM's W8A8 GEMM), blog.gitcode.com.
 *
 * Conventions shared by every entry point
 *   - Shapes follow [LQ]'s notation: X is [M][K] (M tokens, K input
 *     channels), W is [N][K] (N output channels, nn.Linear.weight layout),
 *     Y is [M][N].  All matrices are dense row-major with no padding.
 *   - Functions whose name ends in _host, and q4_pack / q4_unpack /
 *     i8_azp_adj, are synchronous CPU functions on host memory.
 *   - Every other function takes DEVICE pointers (memory of the current HIP
 *     device) and a hipStream_t passed as `void* stream` (NULL = the null
 *     stream).  It validates its arguments on the host, then enqueues its
 *     kernels and returns without synchronizing.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     retains device memory, and keeps no device state between calls
 *     (scratch space comes in as a caller-owned workspace argument).
 *   - Every function returns a ql_status.  Nothing aborts or throws across
 *     the ABI.  On a non-OK return nothing was launched and nothing was
 *     written, and ql_last_error() describes the failure (per thread).
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QL_ABI_VERSION 2

typedef enum {
  QL_OK = 0,
  QL_ERR_NULL = -1,         /* a required pointer is NULL                          */
  QL_ERR_SHAPE = -2,        /* a size is negative, zero where not allowed, or inconsistent */
  QL_ERR_DTYPE = -3,        /* unknown ql_dtype                                    */
  QL_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned                    */
  QL_ERR_UNSUPPORTED = -5,  /* a valid request this build does not implement       */
  QL_ERR_SIZE = -6,         /* a buffer is smaller than the shape requires         */
  QL_ERR_HIP = -7,          /* the HIP runtime reported an error at launch          */
  QL_ERR_RANGE = -8         /* an input value is outside the representable range   */
} ql_status;

typedef enum { QL_F16 = 0, QL_BF16 = 1 } ql_dtype;

/* Message of the last non-OK return on the calling thread ("" if none). */
const char* ql_last_error(void);

/* QL_ABI_VERSION of the loaded library. */
int ql_abi_version(void);

/* =========================================================================
 * W4A16 — offline weight preparation (host, CPU)
 * ========================================================================= */

/*
 * q4_quantize_host — per-group asymmetric round-to-nearest to uint4.
 *
 * [QK] §9.3 (granularity: g = 128 consecutive input channels share a scale)
 * and [LQ] "粒度" (granularity); [LQ] "对称与非对称" (asymmetric uint4 codes
 * 0..15 with a zero point, the GPTQ/AWQ storage convention); the scale and
 * zero point of a range from [LQ] "线性量化：一把刻度尺".  For each output
 * channel n and group g, in IEEE fp32 with round-half-to-even:
 *     mn = min(min w, 0), mx = max(max w, 0)
 *     s  = fp16(max(mx − mn, 1e-5) / 15)
 *     z  = clamp(round(−mn / s), 0, 15)
 *     q  = clamp(round(w / s) + z, 0, 15)
 * (the codes use the fp16-rounded scale, so the stored triple is consistent).
 *
 * W       [N][K] fp32, host.
 * wq      [K/8][N] uint32 out: canonical packing, 8 codes along K per word,
 *         the code of k = 8j + i at bits 4i..4i+3 of wq[j][n] ([LQ] W4A16
 *         section: [11, 6, 15, 0, 3, 9, 12, 7] packs to 0x7C930F6B).
 * scales  [K/group][N] fp16 bit patterns out.
 * zeros   [K/group][N] uint8 out, values 0..15.
 * Errors: QL_ERR_NULL; QL_ERR_SHAPE unless N > 0, K > 0, K % group == 0;
 *         QL_ERR_UNSUPPORTED unless group == 128;
 *         QL_ERR_RANGE if a group's range overflows the fp16 scale or W holds NaN.
 */
int q4_quantize_host(const float* W, int N, int K, int group,
                     uint32_t* wq, uint16_t* scales, uint8_t* zeros);

/*
 * q4_quantize_sym_host — per-group symmetric round-to-nearest to 4 bits with
 * the zero point fixed at 8 (unsigned codes 1..15 standing for −7..7).
 *
 * [LQ] "对称与非对称": z = 0, s = max|w| / q_max with q_max = 7, signed codes
 * −7..7 (−8 unused); stored as the unsigned code + 8, which is exactly the
 * asymmetric code of a zero point 8 ([QK] §9.5's plain decode subtracts 8).
 * For each output channel n and group g, in IEEE fp32 with round-half-to-even:
 *     s = fp16(max(max |w|, 1e-5) / 7),  q = clamp(round(w / s), −7, 7) + 8
 * No zero-point array: pass zeros = NULL to q4_pack.
 * W [N][K] fp32; wq [K/8][N] canonical words out; scales [K/group][N] fp16 out.
 * Errors: as q4_quantize_host.
 */
int q4_quantize_sym_host(const float* W, int N, int K, int group, uint32_t* wq, uint16_t* scales);

/*
 * q4_packed_bytes — size of the device weight blob for an N x K layer.
 * Returns 0 for invalid sizes (see q4_pack).
 */
size_t q4_packed_bytes(int N, int K, int group);

/*
 * q4_pack — canonical (wq, scales, zeros) to the gfx950 device blob (host).
 *
 * The blob keeps the int4 codes packed (the fused kernel reads only packed
 * codes; [QK] §9.5) in an order chosen so that one 16-byte load per lane
 * feeds the in-register unpack with no shuffles; kernels of other projects
 * use other interleaves for the same reason ([LQ] W4A16 section), so blobs
 * are not interchangeable with other formats.  Layout (N and K padded to
 * Np = roundup(N, 64), Kp = roundup(K, 256) with code 0, scale 0, zero 0):
 *   [0, 256)      header: "QL4P", version 2, N, K, group, Np, Kp
 *   weights       [Kp/32][Np][16 bytes]: row c holds, for each output channel
 *                 n, its 32 codes of k in [32c, 32c + 32) as 4 words of 8
 *                 codes, the code of k = 32c + 8j + i sitting at nibble
 *                 position (i & 1) * 4 + (i >> 1) of word j (so that one AND
 *                 with 0x000F000F after a shift by 4p yields the codes of
 *                 k = 8j + 2p and 8j + 2p + 1 as two 16-bit lanes)
 *   scales        [Kp/256][Np][2] fp16: the scales of groups 2p and 2p + 1
 *   zeros         [Kp/256][Np] bytes: zero of group 2p in the low nibble,
 *                 of group 2p + 1 in the high nibble
 * (each region starts on a 256-byte boundary).  The rows are chunk-major so
 * that all output channels at one K position are contiguous in memory.
 *
 * zeros == NULL stores the zero point 8 for every group (the symmetric codes
 * of q4_quantize_sym_host).
 * packed: host buffer of packed_bytes >= q4_packed_bytes(N, K, group).
 * Copy it to device memory (any 16-byte-aligned address) for q4_gemm.
 * Errors: QL_ERR_NULL (wq, scales or packed); QL_ERR_SHAPE as q4_quantize_host;
 *         QL_ERR_UNSUPPORTED unless group == 128; QL_ERR_SIZE if packed_bytes is too small;
 *         QL_ERR_RANGE if a code or zero exceeds 15.
 */
int q4_pack(const uint32_t* wq, const uint16_t* scales, const uint8_t* zeros,
            int N, int K, int group, void* packed, size_t packed_bytes);

/*
 * q4_unpack — inverse of q4_pack (host), for round-trip checks.
 * Errors: as q4_pack; QL_ERR_SHAPE if the blob header disagrees with (N, K, group).
 */
int q4_unpack(const void* packed, size_t packed_bytes, int N, int K, int group,
              uint32_t* wq, uint16_t* scales, uint8_t* zeros);

/* =========================================================================
 * W4A16 — forward (device)
 * ========================================================================= */

/*
 * q4_gemm — Y = X · dequant(W)ᵀ with the dequantization fused into the product.
 *
 * Y[m][n] = Σ_k X[m][k] · s[k/128][n] · (q[n][k] − z[k/128][n]), fp32
 * accumulation, one round-to-nearest-even to x_dtype at the store
 * ([QK] §9.5 "关键 Kernel: Dequant + GEMM": INT4 stays packed in HBM and
 * on chip and is expanded in registers right before the multiply; [LQ]
 * W4A16 section and its tiled pseudocode; the scale rule of [LQ]
 * "哪些 scale 能提到求和号外面": per-group scales along K are fine because
 * the weights are expanded before the multiply).
 *
 * X       [M][K] fp16 or bf16 (x_dtype), device.
 * packed  device blob from q4_pack for (N, K, group), of packed_bytes bytes
 *         (at least q4_packed_bytes(N, K, group)).
 * Y       [M][N] out, same dtype as X, device.
 * workspace, ws_bytes  caller-owned device scratch for a split of K across
 *         workgroups (fp32 partial results, then a pass that adds them and
 *         rounds once to x_dtype), or NULL.  q4_gemm_workspace_bytes gives the
 *         size; NULL runs the layer without a K split (same result up to the
 *         fp32 summation order, possibly slower).  Its contents on entry do
 *         not matter; calls that share one workspace must not overlap.
 * M <= 16 runs the decode kernel (each workgroup owns 16 * NT output
 * channels for all of K); larger M the LDS-tiled MFMA GEMM, with K split
 * across workgroups when few tokens would leave compute units idle.
 * M == 0 or N == 0 is a no-op returning QL_OK.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M, N >= 0, K > 0,
 *         K % group == 0; QL_ERR_UNSUPPORTED unless group == 128, and for
 *         M > 16 when X (M*K*2 bytes) or the blob exceeds 4 GiB;
 *         QL_ERR_SIZE if packed_bytes < q4_packed_bytes(N, K, group) or a
 *         workspace is given with ws_bytes < q4_gemm_workspace_bytes(M, N, K,
 *         group); QL_ERR_ALIGN; QL_ERR_HIP.
 */
int q4_gemm(const void* X, int x_dtype, int M, int K, int N,
            const void* packed, size_t packed_bytes, int group, void* Y,
            void* workspace, size_t ws_bytes, void* stream);

/*
 * q4_gemm_no_alloc — q4_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same plan and kernels as q4_gemm with a workspace, the
 * K-split partials kept in a static device array of the library
 * (32 MiB per device, held until the process ends; looked up once per device
 * on the first call there).  Allocates nothing and calls no allocating
 * routine.  Every call on one device shares that array: calls that overlap
 * on one device (other streams, other threads) race and must not be issued.
 * Nothing in the array needs clearing: every partial is written before it is
 * read.  Arguments as q4_gemm without the workspace.
 * Errors: as q4_gemm; QL_ERR_SIZE also when the layer's plan needs more
 *         scratch than the library holds (more than 32 MiB: q4_gemm with a
 *         workspace serves it).
 */
int q4_gemm_no_alloc(const void* X, int x_dtype, int M, int K, int N,
                     const void* packed, size_t packed_bytes, int group, void* Y, void* stream);

/*
 * q4_gemm_workspace_bytes — bytes of workspace q4_gemm uses for an M x N x K
 * layer (host; 0 when its plan does not split K, and for invalid sizes).
 */
size_t q4_gemm_workspace_bytes(int M, int N, int K, int group);

/*
 * q4_gemm_tile_shape — the plan q4_gemm uses for an M x N x K product, with
 * a workspace (with_workspace != 0) or without one (host; a diagnostic for
 * tests and tuning, no device work).
 * *rows, *cols: the workgroup tile (256 x 256 … 32 x 32, also 128 x 256,
 * 64 x 128 and 32 x 64) for M > 16; 0, 0 for M <= 16 (the decode kernel).  *splits (if
 * splits != NULL): the number of K splits across workgroups (1 = none).
 * The choice depends on the shape only ([LQ] W4A16 section: the batch size
 * decides between the bandwidth- and compute-bound regimes).
 * Errors: QL_ERR_NULL (rows or cols); QL_ERR_SHAPE unless M >= 0, N > 0,
 *         K > 0, K % 128 == 0.
 */
int q4_gemm_tile_shape(int M, int N, int K, int with_workspace, int* rows, int* cols, int* splits);

/* -------------------------------------------------------------------------
 * Act-order (g_idx).  [LQ] GPTQ section, "工程细节", its act-order item:
 * input channels are quantized in decreasing activation energy, groups are
 * formed along that processing order, and g_idx[k] records the group of
 * input channel k, so the scale of a channel is no longer found at k / group.
 * Here the blob is stored in processing order (every group is again a run of
 * `group` channels) together with the permutation perm (perm[j] = the
 * original channel at position j), and the activations are permuted once per
 * call: Y = X · Wᵀ = Xp · Wpᵀ with Xp[m][j] = X[m][perm[j]].  Forward:
 * q4_permute_columns(X → Xp), then q4_gemm(Xp, blob).
 * ------------------------------------------------------------------------- */

/*
 * q4_quantize_act_order_host — q4_quantize_host with the groups given by
 * g_idx (host): group g holds the channels k with g_idx[k] == g, and its
 * (scale, zero) come from those channels' weights by the same formulas.
 * g_idx [K] int32: every value in [0, K/group) and every group holding
 * exactly `group` channels.  wq / scales / zeros as q4_quantize_host (codes in
 * the original channel order, scales and zeros indexed by group).
 * Errors: as q4_quantize_host; QL_ERR_RANGE for an invalid g_idx.
 */
int q4_quantize_act_order_host(const float* W, int N, int K, int group, const int32_t* g_idx,
                               uint32_t* wq, uint16_t* scales, uint8_t* zeros);

/*
 * q4_pack_act_order — q4_pack of the codes reordered into processing order
 * (host).  perm [K] int32 out: perm[j] = the channel whose code sits at
 * position j (the channels of group g, ascending, at positions g·group ..
 * g·group + group − 1).  Copy perm to the device for q4_permute_columns.
 * Errors: as q4_pack; QL_ERR_NULL also for g_idx or perm; QL_ERR_RANGE for an
 *         invalid g_idx.
 */
int q4_pack_act_order(const uint32_t* wq, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* g_idx, int N, int K, int group,
                      void* packed, size_t packed_bytes, int32_t* perm);

/*
 * q4_permute_columns — Xp[m][j] = X[m][perm[j]] (device), the activations in
 * the blob's channel order.  X and Xp [M][K] fp16/bf16 (distinct buffers);
 * perm [K] int32 on the device (values outside [0, K) are clamped: wrong
 * output, never an out-of-bounds read).  M == 0 is a no-op.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M >= 0, K > 0 and
 *         K % 8 == 0; QL_ERR_UNSUPPORTED if M > 65535 or X == Xp;
 *         QL_ERR_ALIGN; QL_ERR_HIP.
 */
int q4_permute_columns(const void* X, int x_dtype, int M, int K, const int32_t* perm,
                       void* Xp, void* stream);

/* =========================================================================
 * W8A8
 * ========================================================================= */

/*
 * i8_quant_weight_host — symmetric per-output-channel int8 weights (host).
 * [LQ] "对称与非对称" (s = max|w| / 127, codes −127..127) and [LQ] W8A8
 * section (weights per channel); [VE] "一、背景" (weights symmetric only).
 * In IEEE fp32: s_b[n] = max(max_k |W[n][k]|, 1e-5) / 127,
 *               Bq[n][k] = clamp(round(W[n][k] / s_b[n]), −127, 127).
 * W [N][K] fp32; Bq [N][K] int8 out (the [N][K] rows are the columns of
 * the page's column-major b); s_b [N] fp32 out.
 * Errors: QL_ERR_NULL; QL_ERR_SHAPE unless N > 0, K > 0; QL_ERR_RANGE on NaN/inf.
 */
int i8_quant_weight_host(const float* W, int N, int K, int8_t* Bq, float* s_b);

/*
 * i8_azp_adj — azp_adj[n] = Σ_k Bq[n][k] (host), the row vector 1 · B̂ that
 * every row of J_a · B̂ equals ([VE] "二、底层线性代数推导" and
 * "五、azp_adj 的离线预计算": independent of scales and zero points, computed
 * once when the weights are loaded).  For a per-tensor zero point the caller
 * multiplies it by z_a itself ([VE] "2.3").
 * Errors: QL_ERR_NULL; QL_ERR_SHAPE; QL_ERR_RANGE if a sum leaves int32.
 */
int i8_azp_adj(const int8_t* Bq, int N, int K, int32_t* azp_adj);

/*
 * i8_quant_per_token — dynamic per-token int8 activation quantization (device).
 *
 * Asymmetric (azp != NULL), per row m in IEEE fp32, round-half-to-even
 * ([LQ] "线性量化" for (s, z) of a range; [LQ] "校准：静态与动态": per-token
 * dynamic ranges at run time; int8 range [−128, 127] from [QK] §9.2; azp
 * int32 per row from [VE] "4.1"):
 *     mn = min(min_k x, 0), mx = max(max_k x, 0)
 *     s_a[m] = max(mx − mn, 1e-5) / 255
 *     azp[m] = −128 − round(mn / s_a[m])
 *     Aq[m][k] = clamp(round(x / s_a[m]) + azp[m], −128, 127)
 * Symmetric (azp == NULL): s_a = max(max_k |x|, 1e-5) / 127,
 *     Aq = clamp(round(x / s_a), −127, 127).
 * The division is a correctly rounded fp32 division, so codes are bit-exact
 * with any IEEE implementation of the same steps.
 *
 * X [M][K] fp16/bf16; Aq [M][K] int8 out; s_a [M] fp32 out; azp [M] int32
 * out or NULL.  M == 0 is a no-op.  A row holding a NaN gets an unspecified
 * scale, zero point and codes.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M >= 0, K > 0 and
 *         K % 8 == 0; QL_ERR_ALIGN; QL_ERR_HIP.
 */
int i8_quant_per_token(const void* X, int x_dtype, int M, int K,
                       int8_t* Aq, float* s_a, int32_t* azp, void* stream);

/*
 * i8_rmsnorm_quant_per_token — RMSNorm fused with the dynamic per-token int8
 * quantization of its output (device).  The normalized activations are never
 * written: the kernel that normalizes a row also takes its range and emits
 * its codes ([QK] §9.9: fuse the per-row reduction of the activation
 * quantization into the producing operator; [LQ] "校准：静态与动态": the
 * per-token reduction is folded into RMSNorm; RMSNorm as x / rms(x) · γ from
 * [LQ] "QuaRot：把整个残差流旋转掉" and "缩放融合到哪里").
 *
 * Per row m, in this order (IEEE, round-half-to-even):
 *     ms  = fp32( (Σ_k x² in fp64) / K in fp64 )      (the squares are exact)
 *     inv = 1 / sqrt(ms + eps)                          (fp32, correctly rounded)
 *     y   = (x · inv) · gamma[k]                        (fp32; not rounded to 16 bits)
 * then y is quantized exactly as i8_quant_per_token quantizes x: asymmetric
 * with azp != NULL, symmetric with azp == NULL.
 *
 * X [M][K] fp16/bf16; gamma [K] of the same dtype; eps > 0 and finite; Aq
 * [M][K] int8 out; s_a [M] fp32 out; azp [M] int32 out or NULL.  M == 0 is a
 * no-op.  Inputs are read once; nothing is allocated.  A row whose
 * normalized values hold a NaN gets an unspecified scale, zero point and codes.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M >= 0, K > 0 and
 *         K % 8 == 0; QL_ERR_RANGE unless eps > 0 and finite; QL_ERR_ALIGN;
 *         QL_ERR_HIP.
 */
int i8_rmsnorm_quant_per_token(const void* X, int x_dtype, int M, int K,
                               const void* gamma, float eps,
                               int8_t* Aq, float* s_a, int32_t* azp, void* stream);

/*
 * i8_gemm_scaled — int8 GEMM with int32 accumulation and the fused epilogue
 * (device).
 *
 * Dq[m][n] = Σ_k Aq[m][k] · Bq[n][k]                       (int32)
 * C[m][n]  = Dq − azp[m] · azp_adj[n]   if azp != NULL      ([VE] "2.4")
 *          = Dq − azp_adj[n]            if azp == NULL, azp_adj != NULL
 *                                       (azp_adj = z_a · 1·B̂, [VE] "2.3")
 *          = Dq                         if both NULL        ([VE] "2.1", "2.2")
 * out[m][n] = s_a[m] · (s_b[n] · float(C)) + bias[n]   (fp32; bias NULL → 0),
 *             one round-to-nearest-even to out_dtype at the single store
 * ([LQ] W8A8 section; [VE] "一、背景": fusing the scale and zero-point
 * correction avoids writing and re-reading the int32 result; [VE] "3.4":
 * the correction is a rank-1 term, O(M + N) memory).  C is exact while
 * |C| < 2^31 (the int32 accumulator wraps beyond that).
 *
 * Aq [M][K] int8 row-major; Bq [N][K] int8 (each row one output channel;
 * the page's column-major b).  s_a: s_a_len == 1 (per tensor) or M (per
 * token); s_b: s_b_len == 1 or N (per channel) ([VE] "4.1").  azp [M] int32
 * or NULL; azp_adj [N] int32 or NULL; bias [N] of out_dtype or NULL ([VE]
 * "4.1": bias dtype equals the output dtype).  out [M][N] of out_dtype.
 * raw_out: optional [M][N] int32 that receives C (for exact checks), or NULL.
 * Few tokens (M <= 16, or M <= 64 with M * N <= 2^19) run a kernel that
 * streams Bq once per block of output channels; larger M the LDS-tiled MFMA
 * GEMM.  Both give the same C.
 * M == 0 or N == 0 is a no-op.
 * Errors: QL_ERR_NULL (also azp without azp_adj); QL_ERR_DTYPE; QL_ERR_SHAPE
 *         unless M, N >= 0, K > 0, K % 16 == 0, s_a_len in {1, M},
 *         s_b_len in {1, N}; QL_ERR_ALIGN; QL_ERR_HIP.
 */
int i8_gemm_scaled(const int8_t* Aq, const int8_t* Bq, int M, int N, int K,
                   const float* s_a, int s_a_len, const float* s_b, int s_b_len,
                   const int32_t* azp, const int32_t* azp_adj, const void* bias,
                   void* out, int out_dtype, int32_t* raw_out, void* stream);

/* =========================================================================
 * W8A8 with FP8 (E4M3) codes
 * ========================================================================= */

/*
 * FP8 E4M3 as in [LQ] "浮点：指数管范围，尾数管精度": the "FN" variant (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits), no infinities, only
 * S.1111.111 is NaN, largest finite value 1.75 · 2^8 = 448; conversion
 * rounds to nearest even and saturates (the page converts 500 to 448).
 * The W8A8 route of [LQ] "W4A4、FP8 与块缩放格式": x / s is converted to
 * E4M3 instead of being rounded to an int8 code, the FP8 products are
 * accumulated in fp32 and the epilogue multiplies the two scales; scales are
 * per token for activations and per channel for weights.  Scale: the absmax
 * maps to the largest code, s = max(absmax, 1e-5) / 448, in IEEE fp32.
 */

/*
 * f8_quant_weight_host — per-output-channel FP8 weights (host).
 * s_b[n] = max(max_k |W[n][k]|, 1e-5) / 448, Bq[n][k] = e4m3(W[n][k] / s_b[n]).
 * W [N][K] fp32; Bq [N][K] E4M3 codes out; s_b [N] fp32 out.
 * Errors: QL_ERR_NULL; QL_ERR_SHAPE unless N > 0, K > 0; QL_ERR_RANGE on NaN/inf.
 */
int f8_quant_weight_host(const float* W, int N, int K, uint8_t* Bq, float* s_b);

/*
 * f8_quant_per_token — dynamic per-token FP8 activation quantization (device).
 * s_a[m] = max(max_k |X[m][k]|, 1e-5) / 448, Aq[m][k] = e4m3(X[m][k] / s_a[m])
 * (correctly rounded fp32 division, then one E4M3 rounding: bit-exact with
 * any IEEE implementation of the same steps).
 * X [M][K] fp16/bf16; Aq [M][K] E4M3 codes out; s_a [M] fp32 out.
 * M == 0 is a no-op.  A row holding a NaN gets an unspecified scale and codes.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M >= 0, K > 0 and
 *         K % 8 == 0; QL_ERR_ALIGN; QL_ERR_HIP.
 */
int f8_quant_per_token(const void* X, int x_dtype, int M, int K, uint8_t* Aq, float* s_a, void* stream);

/*
 * f8_gemm_scaled — FP8 GEMM with fp32 accumulation and the fused epilogue
 * (device).
 * out[m][n] = s_a[m] · (s_b[n] · Σ_k e4m3(Aq[m][k]) · e4m3(Bq[n][k])) + bias[n],
 * one round-to-nearest-even to out_dtype at the single store.
 * Aq [M][K] and Bq [N][K] E4M3 codes (NaN codes are not allowed); s_a:
 * s_a_len 1 or M; s_b: s_b_len 1 or N; bias [N] of out_dtype or NULL;
 * out [M][N] of out_dtype.  M == 0 or N == 0 is a no-op.  The same two
 * kernels as i8_gemm_scaled (chosen by the same rule); the fp32 sums of the
 * two differ only in their order.
 * Errors: QL_ERR_NULL; QL_ERR_DTYPE; QL_ERR_SHAPE unless M, N >= 0, K > 0,
 *         K % 16 == 0, s_a_len in {1, M}, s_b_len in {1, N}; QL_ERR_ALIGN;
 *         QL_ERR_HIP.
 */
int f8_gemm_scaled(const uint8_t* Aq, const uint8_t* Bq, int M, int N, int K,
                   const float* s_a, int s_a_len, const float* s_b, int s_b_len,
                   const void* bias, void* out, int out_dtype, void* stream);

/* =========================================================================
 * Measurement aid
 * ========================================================================= */

/*
 * ql_read_probe — a plain streaming read of `bytes` bytes at src (device):
 * the achievable HBM read rate on this part, against which the decode kernel
 * is measured in the same run ([QK] §9.1: batch-1 decode reads every weight
 * once per token, so its time is at least the weight bytes over the memory
 * bandwidth; [LQ] "带宽与算力：Roofline").  workgroups: grid size in
 * [1, 65536] of 256 threads; mode 0: every thread reads 16-byte pieces at
 * the grid stride; mode 1: every workgroup reads one contiguous chunk of
 * bytes / workgroups.  Non-temporal 16-byte loads, 8 in flight per thread.
 * sink: device buffer of 4 * workgroups uint32 words, overwritten with an XOR
 * of the bytes read (so the loads cannot be elided).  Nothing else is
 * written.
 * Errors: QL_ERR_SHAPE unless bytes is a positive multiple of 16, workgroups
 *         in range and mode 0 or 1; QL_ERR_NULL; QL_ERR_ALIGN; QL_ERR_HIP.
 */
int ql_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, int mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
