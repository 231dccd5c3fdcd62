// The C ABI of libqlinear.so: argument validation on the host, then one or
// more asynchronous launches on the caller's stream.  No allocation, no
// synchronization, no device state.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <string>

#include "../../include/qlinear.h"
#include "ql_internal.h"

namespace ql {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace ql

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return QL_OK;
  return ql::set_error(QL_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

bool valid_dtype(int d) { return d == QL_F16 || d == QL_BF16; }

}  // namespace

extern "C" {

const char* ql_last_error(void) { return ql::g_last_error.c_str(); }

int ql_abi_version(void) { return QL_ABI_VERSION; }

namespace {

// checks shared by q4_gemm and q4_gemm_no_alloc; on QL_OK with *run set the
// layer is non-empty and its blob layout is in *L
int q4_gemm_check(const char* fn, const void* X, int x_dtype, int M, int K, int N, const void* packed,
                  size_t packed_bytes, int group, const void* Y, ql::Q4Layout* L, bool* run) {
  *run = false;
  if (M < 0 || N < 0 || K <= 0)
    return ql::set_error(QL_ERR_SHAPE, "%s: need M >= 0, N >= 0, K > 0 (got %d, %d, %d)", fn, M, N, K);
  if (group != ql::kGroup)
    return ql::set_error(QL_ERR_UNSUPPORTED, "%s: group=%d; this build supports group=128", fn, group);
  if (K % group) return ql::set_error(QL_ERR_SHAPE, "%s: K=%d is not a multiple of group=%d", fn, K, group);
  if (!valid_dtype(x_dtype)) return ql::set_error(QL_ERR_DTYPE, "%s: x_dtype=%d", fn, x_dtype);
  if (M == 0 || N == 0) return QL_OK;
  if (!X || !packed || !Y) return ql::set_error(QL_ERR_NULL, "%s: NULL X, packed or Y", fn);
  if (!aligned16(X) || !aligned16(packed) || !aligned16(Y))
    return ql::set_error(QL_ERR_ALIGN, "%s: X, packed and Y must be 16-byte aligned", fn);
  *L = ql::q4_layout(N, K);
  if (packed_bytes < L->bytes)
    return ql::set_error(QL_ERR_SIZE, "%s: packed_bytes=%zu < %zu for N=%d K=%d", fn, packed_bytes, L->bytes, N, K);
  // the large-M kernel addresses X and the weights with 32-bit byte offsets
  if (M > ql::kGemvMaxM && ((size_t)M * K * 2 > 0xFFFFFFFFu || L->bytes > 0xFFFFFFFFu))
    return ql::set_error(QL_ERR_UNSUPPORTED, "%s: M*K*2 = %zu bytes or a packed blob of %zu bytes exceeds 4 GiB", fn,
                         (size_t)M * K * 2, L->bytes);
  *run = true;
  return QL_OK;
}

// launches a checked layer; ws: the plan's workspace (null: no K split)
int q4_gemm_launch(const char* fn, const void* X, int x_dtype, int M, int K, int N, const void* packed,
                   const ql::Q4Layout& L, void* Y, const ql::GemmPlan* plan, float* ws, hipStream_t st) {
  const bool bf16 = x_dtype == QL_BF16;
  const uint8_t* blob = static_cast<const uint8_t*>(packed);
  if (M <= ql::kGemvMaxM)
    return hip_status(fn, ql::launch_q4_gemv(X, bf16, M, K, N, blob, L, ql::plan_q4_gemv(M, N, K), Y, st));
  return hip_status(fn, ql::launch_q4_gemm(X, bf16, M, K, N, blob, L, *plan, Y, ws, st));
}

}  // namespace

size_t q4_gemm_workspace_bytes(int M, int N, int K, int group) {
  if (M <= ql::kGemvMaxM || N <= 0 || K <= 0 || group != ql::kGroup || K % group) return 0;
  return ql::gemm_workspace_bytes(ql::plan_q4_gemm(M, N, K, 8), M, N);
}

int q4_gemm(const void* X, int x_dtype, int M, int K, int N, const void* packed, size_t packed_bytes, int group,
            void* Y, void* workspace, size_t ws_bytes, void* stream) {
  ql::Q4Layout L;
  bool run;
  const int rc = q4_gemm_check("q4_gemm", X, x_dtype, M, K, N, packed, packed_bytes, group, Y, &L, &run);
  if (rc != QL_OK || !run) return rc;
  if (workspace && !aligned16(workspace))
    return ql::set_error(QL_ERR_ALIGN, "q4_gemm: the workspace must be 16-byte aligned");
  ql::GemmPlan plan{0, 1, 0};
  if (M > ql::kGemvMaxM) {
    // without a workspace the layer runs unsplit (a valid, possibly slower plan)
    plan = ql::plan_q4_gemm(M, N, K, workspace ? 8 : 1);
    const size_t need = ql::gemm_workspace_bytes(plan, M, N);
    if (ws_bytes < need)
      return ql::set_error(QL_ERR_SIZE, "q4_gemm: ws_bytes=%zu < %zu (q4_gemm_workspace_bytes) for M=%d N=%d K=%d",
                           ws_bytes, need, M, N, K);
  }
  return q4_gemm_launch("q4_gemm", X, x_dtype, M, K, N, packed, L, Y, &plan, static_cast<float*>(workspace),
                        static_cast<hipStream_t>(stream));
}

int q4_gemm_no_alloc(const void* X, int x_dtype, int M, int K, int N, const void* packed, size_t packed_bytes,
                     int group, void* Y, void* stream) {
  ql::Q4Layout L;
  bool run;
  const int rc = q4_gemm_check("q4_gemm_no_alloc", X, x_dtype, M, K, N, packed, packed_bytes, group, Y, &L, &run);
  if (rc != QL_OK || !run) return rc;
  ql::GemmPlan plan{0, 1, 0};
  void* ws = nullptr;
  if (M > ql::kGemvMaxM) {
    plan = ql::plan_q4_gemm(M, N, K, 8);                 // the plan q4_gemm runs with a workspace
    const size_t need = ql::gemm_workspace_bytes(plan, M, N);
    if (need > ql::kStaticScratchBytes)
      return ql::set_error(QL_ERR_SIZE,
                           "q4_gemm_no_alloc: M=%d N=%d K=%d needs %zu bytes of scratch; the library's static "
                           "scratch holds %zu (use q4_gemm with a workspace)",
                           M, N, K, need, ql::kStaticScratchBytes);
    if (need) {
      const int e = hip_status("q4_gemm_no_alloc", ql::static_scratch(&ws));
      if (e != QL_OK) return e;
    }
  }
  return q4_gemm_launch("q4_gemm_no_alloc", X, x_dtype, M, K, N, packed, L, Y, &plan, static_cast<float*>(ws),
                        static_cast<hipStream_t>(stream));
}

int q4_gemm_tile_shape(int M, int N, int K, int with_workspace, int* rows, int* cols, int* splits) {
  if (!rows || !cols) return ql::set_error(QL_ERR_NULL, "q4_gemm_tile_shape: NULL rows or cols");
  if (M < 0 || N <= 0 || K <= 0 || K % ql::kGroup)
    return ql::set_error(QL_ERR_SHAPE, "q4_gemm_tile_shape: need M >= 0, N > 0, K > 0, K %% 128 == 0 (got %d, %d, %d)",
                         M, N, K);
  if (M <= ql::kGemvMaxM) {
    *rows = *cols = 0;
    if (splits) *splits = 1;
    return QL_OK;
  }
  const ql::GemmPlan p = ql::plan_q4_gemm(M, N, K, with_workspace ? 8 : 1);
  ql::gemm_tile_shape(p, rows, cols);
  if (splits) *splits = p.splits;
  return QL_OK;
}

int q4_permute_columns(const void* X, int x_dtype, int M, int K, const int32_t* perm, void* Xp, void* stream) {
  if (M < 0 || K <= 0 || K % 8)
    return ql::set_error(QL_ERR_SHAPE, "q4_permute_columns: need M >= 0, K > 0, K %% 8 == 0 (got %d, %d)", M, K);
  if (!valid_dtype(x_dtype)) return ql::set_error(QL_ERR_DTYPE, "q4_permute_columns: x_dtype=%d", x_dtype);
  if (M == 0) return QL_OK;
  if (M > 65535) return ql::set_error(QL_ERR_UNSUPPORTED, "q4_permute_columns: M=%d exceeds 65535 rows per call", M);
  if (!X || !perm || !Xp) return ql::set_error(QL_ERR_NULL, "q4_permute_columns: NULL X, perm or Xp");
  if (!aligned16(X) || !aligned16(perm) || !aligned16(Xp))
    return ql::set_error(QL_ERR_ALIGN, "q4_permute_columns: pointers must be 16-byte aligned");
  if (X == Xp) return ql::set_error(QL_ERR_UNSUPPORTED, "q4_permute_columns: X and Xp must not be the same buffer");
  return hip_status("q4_permute_columns",
                    ql::launch_permute_cols(X, M, K, perm, Xp, static_cast<hipStream_t>(stream)));
}

int i8_quant_per_token(const void* X, int x_dtype, int M, int K, int8_t* Aq, float* s_a, int32_t* azp,
                       void* stream) {
  if (M < 0 || K <= 0 || K % 8)
    return ql::set_error(QL_ERR_SHAPE, "i8_quant_per_token: need M >= 0, K > 0, K %% 8 == 0 (got %d, %d)", M, K);
  if (!valid_dtype(x_dtype)) return ql::set_error(QL_ERR_DTYPE, "i8_quant_per_token: x_dtype=%d", x_dtype);
  if (M == 0) return QL_OK;
  if (!X || !Aq || !s_a) return ql::set_error(QL_ERR_NULL, "i8_quant_per_token: NULL X, Aq or s_a");
  if (!aligned16(X) || !aligned16(Aq) || !aligned16(s_a) || (azp && !aligned16(azp)))
    return ql::set_error(QL_ERR_ALIGN, "i8_quant_per_token: pointers must be 16-byte aligned");
  return hip_status("i8_quant_per_token",
                    ql::launch_i8_quant(X, x_dtype == QL_BF16, M, K, Aq, s_a, azp, static_cast<hipStream_t>(stream)));
}

int i8_rmsnorm_quant_per_token(const void* X, int x_dtype, int M, int K, const void* gamma, float eps, int8_t* Aq,
                               float* s_a, int32_t* azp, void* stream) {
  if (M < 0 || K <= 0 || K % 8)
    return ql::set_error(QL_ERR_SHAPE, "i8_rmsnorm_quant_per_token: need M >= 0, K > 0, K %% 8 == 0 (got %d, %d)", M,
                         K);
  if (!valid_dtype(x_dtype)) return ql::set_error(QL_ERR_DTYPE, "i8_rmsnorm_quant_per_token: x_dtype=%d", x_dtype);
  if (!(eps > 0.0f) || !std::isfinite(eps))
    return ql::set_error(QL_ERR_RANGE, "i8_rmsnorm_quant_per_token: eps=%g must be > 0 and finite", (double)eps);
  if (M == 0) return QL_OK;
  if (!X || !gamma || !Aq || !s_a) return ql::set_error(QL_ERR_NULL, "i8_rmsnorm_quant_per_token: NULL X, gamma, Aq or s_a");
  if (!aligned16(X) || !aligned16(gamma) || !aligned16(Aq) || !aligned16(s_a) || (azp && !aligned16(azp)))
    return ql::set_error(QL_ERR_ALIGN, "i8_rmsnorm_quant_per_token: pointers must be 16-byte aligned");
  return hip_status("i8_rmsnorm_quant_per_token",
                    ql::launch_rmsnorm_quant(X, x_dtype == QL_BF16, M, K, gamma, eps, Aq, s_a, azp,
                                             static_cast<hipStream_t>(stream)));
}

int i8_gemm_scaled(const int8_t* Aq, const int8_t* Bq, int M, int N, int K, const float* s_a, int s_a_len,
                   const float* s_b, int s_b_len, const int32_t* azp, const int32_t* azp_adj, const void* bias,
                   void* out, int out_dtype, int32_t* raw_out, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16)
    return ql::set_error(QL_ERR_SHAPE, "i8_gemm_scaled: need M, N >= 0, K > 0, K %% 16 == 0 (got %d, %d, %d)", M, N, K);
  if (!valid_dtype(out_dtype)) return ql::set_error(QL_ERR_DTYPE, "i8_gemm_scaled: out_dtype=%d", out_dtype);
  if (M == 0 || N == 0) return QL_OK;
  if (s_a_len != 1 && s_a_len != M)
    return ql::set_error(QL_ERR_SHAPE, "i8_gemm_scaled: s_a_len=%d must be 1 or M=%d", s_a_len, M);
  if (s_b_len != 1 && s_b_len != N)
    return ql::set_error(QL_ERR_SHAPE, "i8_gemm_scaled: s_b_len=%d must be 1 or N=%d", s_b_len, N);
  if (!Aq || !Bq || !s_a || !s_b || !out) return ql::set_error(QL_ERR_NULL, "i8_gemm_scaled: NULL operand");
  if (azp && !azp_adj) return ql::set_error(QL_ERR_NULL, "i8_gemm_scaled: azp given without azp_adj");
  const void* ptrs[] = {Aq, Bq, s_a, s_b, azp, azp_adj, bias, out, raw_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ql::set_error(QL_ERR_ALIGN, "i8_gemm_scaled: pointers must be 16-byte aligned");
  ql::I8Epi e{s_a, s_a_len != 1, s_b, s_b_len != 1, azp, azp_adj, bias, out, out_dtype == QL_BF16, raw_out};
  return hip_status("i8_gemm_scaled", ql::launch_i8_gemm(Aq, Bq, M, N, K, e, static_cast<hipStream_t>(stream)));
}

int f8_quant_per_token(const void* X, int x_dtype, int M, int K, uint8_t* Aq, float* s_a, void* stream) {
  if (M < 0 || K <= 0 || K % 8)
    return ql::set_error(QL_ERR_SHAPE, "f8_quant_per_token: need M >= 0, K > 0, K %% 8 == 0 (got %d, %d)", M, K);
  if (!valid_dtype(x_dtype)) return ql::set_error(QL_ERR_DTYPE, "f8_quant_per_token: x_dtype=%d", x_dtype);
  if (M == 0) return QL_OK;
  if (!X || !Aq || !s_a) return ql::set_error(QL_ERR_NULL, "f8_quant_per_token: NULL X, Aq or s_a");
  if (!aligned16(X) || !aligned16(Aq) || !aligned16(s_a))
    return ql::set_error(QL_ERR_ALIGN, "f8_quant_per_token: pointers must be 16-byte aligned");
  return hip_status("f8_quant_per_token",
                    ql::launch_f8_quant(X, x_dtype == QL_BF16, M, K, Aq, s_a, static_cast<hipStream_t>(stream)));
}

int f8_gemm_scaled(const uint8_t* Aq, const uint8_t* Bq, int M, int N, int K, const float* s_a, int s_a_len,
                   const float* s_b, int s_b_len, const void* bias, void* out, int out_dtype, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16)
    return ql::set_error(QL_ERR_SHAPE, "f8_gemm_scaled: need M, N >= 0, K > 0, K %% 16 == 0 (got %d, %d, %d)", M, N, K);
  if (!valid_dtype(out_dtype)) return ql::set_error(QL_ERR_DTYPE, "f8_gemm_scaled: out_dtype=%d", out_dtype);
  if (M == 0 || N == 0) return QL_OK;
  if (s_a_len != 1 && s_a_len != M)
    return ql::set_error(QL_ERR_SHAPE, "f8_gemm_scaled: s_a_len=%d must be 1 or M=%d", s_a_len, M);
  if (s_b_len != 1 && s_b_len != N)
    return ql::set_error(QL_ERR_SHAPE, "f8_gemm_scaled: s_b_len=%d must be 1 or N=%d", s_b_len, N);
  if (!Aq || !Bq || !s_a || !s_b || !out) return ql::set_error(QL_ERR_NULL, "f8_gemm_scaled: NULL operand");
  const void* ptrs[] = {Aq, Bq, s_a, s_b, bias, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ql::set_error(QL_ERR_ALIGN, "f8_gemm_scaled: pointers must be 16-byte aligned");
  ql::I8Epi e{s_a, s_a_len != 1, s_b, s_b_len != 1, nullptr, nullptr, bias, out, out_dtype == QL_BF16, nullptr};
  return hip_status("f8_gemm_scaled", ql::launch_f8_gemm(Aq, Bq, M, N, K, e, static_cast<hipStream_t>(stream)));
}

int ql_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, int mode, void* stream) {
  if (bytes == 0 || bytes % 16)
    return ql::set_error(QL_ERR_SHAPE, "ql_read_probe: bytes=%zu must be a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > 65536)
    return ql::set_error(QL_ERR_SHAPE, "ql_read_probe: workgroups=%d must be in [1, 65536]", workgroups);
  if (mode != 0 && mode != 1) return ql::set_error(QL_ERR_SHAPE, "ql_read_probe: mode=%d must be 0 or 1", mode);
  if (!src || !sink) return ql::set_error(QL_ERR_NULL, "ql_read_probe: NULL src or sink");
  if (!aligned16(src) || !aligned16(sink))
    return ql::set_error(QL_ERR_ALIGN, "ql_read_probe: src and sink must be 16-byte aligned");
  return hip_status("ql_read_probe",
                    ql::launch_read_probe(src, bytes, sink, workgroups, mode, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
