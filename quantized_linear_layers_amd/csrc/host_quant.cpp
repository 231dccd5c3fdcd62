// Offline weight preparation on the CPU: W4 quantize / pack / unpack and the
// int8 weight quantizer and zero-point adjustment.  Plain IEEE fp32 scalar
// code (no FMA contraction, round-half-to-even via rintf) so that every code
// is decided exactly as the formulas in qlinear.h state.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "../../include/qlinear.h"
#include "ql_internal.h"

namespace {

// fp32 -> fp16 bit pattern, round to nearest even (IEEE binary16).
uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                     // below 2^-14: subnormal grid
    float v;
    memcpy(&v, &ax, 4);
    // v * 2^24 is exact (power-of-two scaling); rintf rounds half to even.
    return (uint16_t)(sign | (uint32_t)rintf(v * 16777216.0f));
  }
  const uint32_t r = ax + 0x0FFFu + ((ax >> 13) & 1u);       // round the 13 dropped bits
  return (uint16_t)(sign | ((r >> 13) - (112u << 10)));
}

float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    const uint32_t bits = ((e + 112u) << 23) | (m << 13);
    memcpy(&v, &bits, 4);
  }
  uint32_t b;
  memcpy(&b, &v, 4);
  b |= sign;
  memcpy(&v, &b, 4);
  return v;
}

struct BlobHeader {
  uint32_t magic, version;
  int32_t N, K, group, Np, Kp;
};

int check_q4_shape(const char* fn, int N, int K, int group) {
  if (N <= 0 || K <= 0) return ql::set_error(QL_ERR_SHAPE, "%s: N=%d and K=%d must be > 0", fn, N, K);
  if (group != ql::kGroup)
    return ql::set_error(QL_ERR_UNSUPPORTED, "%s: group=%d; this build supports group=128", fn, group);
  if (K % group) return ql::set_error(QL_ERR_SHAPE, "%s: K=%d is not a multiple of group=%d", fn, K, group);
  return QL_OK;
}

// chunk-major device layout: row c of 32-channel chunks holds one 16-byte
// chunk per output channel; scale / zero rows hold one group pair per channel
inline size_t w_byte(const ql::Q4Layout& L, int n, int k) {
  const int c = k / ql::kChunkK, j = (k % ql::kChunkK) / 8;
  return L.w_off + ((size_t)c * L.Np + n) * 16 + (size_t)j * 4;
}
inline size_t s_byte(const ql::Q4Layout& L, int n, int g) {
  return L.s_off + ((size_t)(g / 2) * L.Np + n) * 4 + (size_t)(g % 2) * 2;
}
inline size_t z_byte(const ql::Q4Layout& L, int n, int g) { return L.z_off + (size_t)(g / 2) * L.Np + n; }

// Channels of every group in ascending order, from a group index per input
// channel; every group must hold exactly `group` channels (the act-order
// layout: groups are runs of `group` channels of the processing order).
int order_from_g_idx(const char* fn, const int32_t* g_idx, int K, int group, int32_t* order) {
  const int G = K / group;
  int* fill = new int[G]();
  for (int k = 0; k < K; ++k) {
    const int g = g_idx[k];
    if (g < 0 || g >= G || fill[g] >= group) {
      delete[] fill;
      return ql::set_error(QL_ERR_RANGE, "%s: g_idx[%d]=%d is out of range or its group holds more than %d channels",
                           fn, k, g, group);
    }
    order[(size_t)g * group + fill[g]++] = k;
  }
  delete[] fill;
  return QL_OK;
}

}  // namespace

extern "C" {

int q4_quantize_host(const float* W, int N, int K, int group, uint32_t* wq, uint16_t* scales,
                     uint8_t* zeros) {
  if (!W || !wq || !scales || !zeros) return ql::set_error(QL_ERR_NULL, "q4_quantize_host: NULL pointer");
  if (int e = check_q4_shape("q4_quantize_host", N, K, group)) return e;
  const int G = K / group;
  memset(wq, 0, sizeof(uint32_t) * (size_t)(K / 8) * N);
  for (int n = 0; n < N; ++n) {
    for (int g = 0; g < G; ++g) {
      const float* w = W + (size_t)n * K + (size_t)g * group;
      float mn = 0.0f, mx = 0.0f;
      for (int i = 0; i < group; ++i) {
        const float v = w[i];
        if (!(v == v) || isinf(v))
          return ql::set_error(QL_ERR_RANGE, "q4_quantize_host: W[%d][%d] is not finite", n, g * group + i);
        mn = std::min(mn, v);
        mx = std::max(mx, v);
      }
      float range = mx - mn;
      if (range < 1e-5f) range = 1e-5f;
      const uint16_t sb = f32_to_f16_bits(range / 15.0f);
      if ((sb & 0x7C00u) == 0x7C00u)
        return ql::set_error(QL_ERR_RANGE, "q4_quantize_host: group (%d,%d) overflows the fp16 scale", n, g);
      const float s = f16_bits_to_f32(sb);
      const float z = std::min(std::max(rintf(-mn / s), 0.0f), 15.0f);
      scales[(size_t)g * N + n] = sb;
      zeros[(size_t)g * N + n] = (uint8_t)z;
      for (int i = 0; i < group; ++i) {
        const float q = std::min(std::max(rintf(w[i] / s) + z, 0.0f), 15.0f);
        const int k = g * group + i;
        wq[(size_t)(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));
      }
    }
  }
  return QL_OK;
}

int q4_quantize_sym_host(const float* W, int N, int K, int group, uint32_t* wq, uint16_t* scales) {
  if (!W || !wq || !scales) return ql::set_error(QL_ERR_NULL, "q4_quantize_sym_host: NULL pointer");
  if (int e = check_q4_shape("q4_quantize_sym_host", N, K, group)) return e;
  const int G = K / group;
  memset(wq, 0, sizeof(uint32_t) * (size_t)(K / 8) * N);
  for (int n = 0; n < N; ++n) {
    for (int g = 0; g < G; ++g) {
      const float* w = W + (size_t)n * K + (size_t)g * group;
      float amax = 0.0f;
      for (int i = 0; i < group; ++i) {
        const float v = w[i];
        if (!(v == v) || isinf(v))
          return ql::set_error(QL_ERR_RANGE, "q4_quantize_sym_host: W[%d][%d] is not finite", n, g * group + i);
        amax = std::max(amax, fabsf(v));
      }
      if (amax < 1e-5f) amax = 1e-5f;
      const uint16_t sb = f32_to_f16_bits(amax / 7.0f);
      if ((sb & 0x7C00u) == 0x7C00u)
        return ql::set_error(QL_ERR_RANGE, "q4_quantize_sym_host: group (%d,%d) overflows the fp16 scale", n, g);
      const float s = f16_bits_to_f32(sb);
      scales[(size_t)g * N + n] = sb;
      for (int i = 0; i < group; ++i) {
        const float q = std::min(std::max(rintf(w[i] / s), -7.0f), 7.0f) + 8.0f;
        const int k = g * group + i;
        wq[(size_t)(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));
      }
    }
  }
  return QL_OK;
}

int q4_quantize_act_order_host(const float* W, int N, int K, int group, const int32_t* g_idx, uint32_t* wq,
                               uint16_t* scales, uint8_t* zeros) {
  if (!W || !g_idx || !wq || !scales || !zeros)
    return ql::set_error(QL_ERR_NULL, "q4_quantize_act_order_host: NULL pointer");
  if (int e = check_q4_shape("q4_quantize_act_order_host", N, K, group)) return e;
  int32_t* order = new int32_t[K];
  if (int e = order_from_g_idx("q4_quantize_act_order_host", g_idx, K, group, order)) {
    delete[] order;
    return e;
  }
  const int G = K / group;
  memset(wq, 0, sizeof(uint32_t) * (size_t)(K / 8) * N);
  int rc = QL_OK;
  for (int n = 0; n < N && rc == QL_OK; ++n) {
    const float* w = W + (size_t)n * K;
    for (int g = 0; g < G && rc == QL_OK; ++g) {
      const int32_t* ch = order + (size_t)g * group;
      float mn = 0.0f, mx = 0.0f;
      for (int i = 0; i < group; ++i) {
        const float v = w[ch[i]];
        if (!(v == v) || isinf(v)) {
          rc = ql::set_error(QL_ERR_RANGE, "q4_quantize_act_order_host: W[%d][%d] is not finite", n, ch[i]);
          break;
        }
        mn = std::min(mn, v);
        mx = std::max(mx, v);
      }
      if (rc != QL_OK) break;
      float range = mx - mn;
      if (range < 1e-5f) range = 1e-5f;
      const uint16_t sb = f32_to_f16_bits(range / 15.0f);
      if ((sb & 0x7C00u) == 0x7C00u) {
        rc = ql::set_error(QL_ERR_RANGE, "q4_quantize_act_order_host: group (%d,%d) overflows the fp16 scale", n, g);
        break;
      }
      const float sc = f16_bits_to_f32(sb);
      const float z = std::min(std::max(rintf(-mn / sc), 0.0f), 15.0f);
      scales[(size_t)g * N + n] = sb;
      zeros[(size_t)g * N + n] = (uint8_t)z;
      for (int i = 0; i < group; ++i) {
        const int k = ch[i];
        const float q = std::min(std::max(rintf(w[k] / sc) + z, 0.0f), 15.0f);
        wq[(size_t)(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));
      }
    }
  }
  delete[] order;
  return rc;
}

size_t q4_packed_bytes(int N, int K, int group) {
  if (N <= 0 || K <= 0 || group != ql::kGroup || K % group) return 0;
  return ql::q4_layout(N, K).bytes;
}

int q4_pack(const uint32_t* wq, const uint16_t* scales, const uint8_t* zeros, int N, int K, int group,
            void* packed, size_t packed_bytes) {
  if (!wq || !scales || !packed) return ql::set_error(QL_ERR_NULL, "q4_pack: NULL pointer");
  if (int e = check_q4_shape("q4_pack", N, K, group)) return e;
  const ql::Q4Layout L = ql::q4_layout(N, K);
  if (packed_bytes < L.bytes)
    return ql::set_error(QL_ERR_SIZE, "q4_pack: packed_bytes=%zu < %zu", packed_bytes, L.bytes);
  const int G = K / group;
  auto zero = [&](int g, int n) -> uint8_t { return zeros ? zeros[(size_t)g * N + n] : (uint8_t)8; };
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      if (zero(g, n) > 15)
        return ql::set_error(QL_ERR_RANGE, "q4_pack: zeros[%d][%d]=%d exceeds 15", g, n, zeros[(size_t)g * N + n]);
  uint8_t* out = static_cast<uint8_t*>(packed);
  memset(out, 0, L.bytes);
  BlobHeader h{ql::kMagic, ql::kVersion, N, K, group, L.Np, L.Kp};
  memcpy(out, &h, sizeof h);
  for (int k = 0; k < K; ++k) {
    const int i = k % 8;
    const int sh_in = 4 * i, sh_out = 4 * ql::nib_pos(i);
    const uint32_t* row = wq + (size_t)(k / 8) * N;
    for (int n = 0; n < N; ++n) {
      const uint32_t code = (row[n] >> sh_in) & 0xFu;
      uint32_t* word = reinterpret_cast<uint32_t*>(out + w_byte(L, n, k));
      *word |= code << sh_out;
    }
  }
  for (int g = 0; g < G; ++g) {
    for (int n = 0; n < N; ++n) {
      memcpy(out + s_byte(L, n, g), &scales[(size_t)g * N + n], 2);
      out[z_byte(L, n, g)] |= (uint8_t)(zero(g, n) << (4 * (g % 2)));
    }
  }
  return QL_OK;
}

int q4_pack_act_order(const uint32_t* wq, const uint16_t* scales, const uint8_t* zeros, const int32_t* g_idx, int N,
                      int K, int group, void* packed, size_t packed_bytes, int32_t* perm) {
  if (!wq || !scales || !g_idx || !packed || !perm) return ql::set_error(QL_ERR_NULL, "q4_pack_act_order: NULL pointer");
  if (int e = check_q4_shape("q4_pack_act_order", N, K, group)) return e;
  if (int e = order_from_g_idx("q4_pack_act_order", g_idx, K, group, perm)) return e;
  // the codes in processing order: position j holds channel perm[j]
  uint32_t* wp = new uint32_t[(size_t)(K / 8) * N]();
  for (int j = 0; j < K; ++j) {
    const int k = perm[j];
    const uint32_t* src = wq + (size_t)(k / 8) * N;
    uint32_t* dst = wp + (size_t)(j / 8) * N;
    for (int n = 0; n < N; ++n) dst[n] |= ((src[n] >> (4 * (k % 8))) & 0xFu) << (4 * (j % 8));
  }
  const int rc = q4_pack(wp, scales, zeros, N, K, group, packed, packed_bytes);
  delete[] wp;
  return rc;
}

int q4_unpack(const void* packed, size_t packed_bytes, int N, int K, int group, uint32_t* wq,
              uint16_t* scales, uint8_t* zeros) {
  if (!packed || !wq || !scales || !zeros) return ql::set_error(QL_ERR_NULL, "q4_unpack: NULL pointer");
  if (int e = check_q4_shape("q4_unpack", N, K, group)) return e;
  const ql::Q4Layout L = ql::q4_layout(N, K);
  if (packed_bytes < L.bytes)
    return ql::set_error(QL_ERR_SIZE, "q4_unpack: packed_bytes=%zu < %zu", packed_bytes, L.bytes);
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  BlobHeader h;
  memcpy(&h, in, sizeof h);
  if (h.magic != ql::kMagic || h.version != ql::kVersion || h.N != N || h.K != K || h.group != group ||
      h.Np != L.Np || h.Kp != L.Kp)
    return ql::set_error(QL_ERR_SHAPE, "q4_unpack: blob header does not describe a (%d, %d, %d) layer", N, K, group);
  memset(wq, 0, sizeof(uint32_t) * (size_t)(K / 8) * N);
  for (int k = 0; k < K; ++k) {
    const int i = k % 8;
    const int sh_in = 4 * ql::nib_pos(i), sh_out = 4 * i;
    uint32_t* row = wq + (size_t)(k / 8) * N;
    for (int n = 0; n < N; ++n) {
      uint32_t word;
      memcpy(&word, in + w_byte(L, n, k), 4);
      row[n] |= ((word >> sh_in) & 0xFu) << sh_out;
    }
  }
  const int G = K / group;
  for (int g = 0; g < G; ++g) {
    for (int n = 0; n < N; ++n) {
      memcpy(&scales[(size_t)g * N + n], in + s_byte(L, n, g), 2);
      zeros[(size_t)g * N + n] = (in[z_byte(L, n, g)] >> (4 * (g % 2))) & 0xFu;
    }
  }
  return QL_OK;
}

int i8_quant_weight_host(const float* W, int N, int K, int8_t* Bq, float* s_b) {
  if (!W || !Bq || !s_b) return ql::set_error(QL_ERR_NULL, "i8_quant_weight_host: NULL pointer");
  if (N <= 0 || K <= 0) return ql::set_error(QL_ERR_SHAPE, "i8_quant_weight_host: N=%d K=%d must be > 0", N, K);
  for (int n = 0; n < N; ++n) {
    const float* w = W + (size_t)n * K;
    float amax = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float v = w[k];
      if (!(v == v) || isinf(v))
        return ql::set_error(QL_ERR_RANGE, "i8_quant_weight_host: W[%d][%d] is not finite", n, k);
      amax = std::max(amax, fabsf(v));
    }
    if (amax < 1e-5f) amax = 1e-5f;
    const float s = amax / 127.0f;
    s_b[n] = s;
    for (int k = 0; k < K; ++k)
      Bq[(size_t)n * K + k] = (int8_t)std::min(std::max(rintf(w[k] / s), -127.0f), 127.0f);
  }
  return QL_OK;
}

int f8_quant_weight_host(const float* W, int N, int K, uint8_t* Bq, float* s_b) {
  if (!W || !Bq || !s_b) return ql::set_error(QL_ERR_NULL, "f8_quant_weight_host: NULL pointer");
  if (N <= 0 || K <= 0) return ql::set_error(QL_ERR_SHAPE, "f8_quant_weight_host: N=%d K=%d must be > 0", N, K);
  for (int n = 0; n < N; ++n) {
    const float* w = W + (size_t)n * K;
    float amax = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float v = w[k];
      if (!(v == v) || isinf(v))
        return ql::set_error(QL_ERR_RANGE, "f8_quant_weight_host: W[%d][%d] is not finite", n, k);
      amax = std::max(amax, fabsf(v));
    }
    if (amax < 1e-5f) amax = 1e-5f;
    const float s = amax / 448.0f;
    s_b[n] = s;
    for (int k = 0; k < K; ++k) Bq[(size_t)n * K + k] = (uint8_t)ql::e4m3_code(w[k] / s);
  }
  return QL_OK;
}

int i8_azp_adj(const int8_t* Bq, int N, int K, int32_t* azp_adj) {
  if (!Bq || !azp_adj) return ql::set_error(QL_ERR_NULL, "i8_azp_adj: NULL pointer");
  if (N <= 0 || K <= 0) return ql::set_error(QL_ERR_SHAPE, "i8_azp_adj: N=%d K=%d must be > 0", N, K);
  for (int n = 0; n < N; ++n) {
    int64_t s = 0;
    for (int k = 0; k < K; ++k) s += Bq[(size_t)n * K + k];
    if (s > INT32_MAX || s < INT32_MIN) return ql::set_error(QL_ERR_RANGE, "i8_azp_adj: row %d sum leaves int32", n);
    azp_adj[n] = (int32_t)s;
  }
  return QL_OK;
}

}  // extern "C"
