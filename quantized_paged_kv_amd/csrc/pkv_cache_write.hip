// pkv_cache_write.hip -- quantise-on-write of new K/V rows into the paged
// cache (gfx950).
//
// ONNX Runtime PR #29912 (PagedAttention), "Summary of Changes": new tokens
// enter the cache through ReshapeAndCache, which quantises them on write
// with k_scale / v_scale at PER_TENSOR or PER_CHANNEL granularity, at the
// slot the slot_mapping input names (the scheduler owns placement).
//
// One thread converts eight consecutive channels of one KV head for a group
// of kTokens tokens: per token a 16-byte FP16 load, the FP32 quotient by the
// scale, the code chosen by round-half-even, and one 8-byte (16-byte for an
// FP16 cache) store.  Consecutive threads take consecutive chunks of a token
// row, so both sides of the copy are coalesced.  The kernel is bound by VALU
// issue as much as by HBM (one wave instruction per CU per clock against a
// few bytes of traffic per element), so each element costs a handful of
// instructions:
//
// Quotient.  q = RN32(x / s) is formed as RN32(RN64(x * RN64(1 / s))) with
// the reciprocal taken once per thread.  That is exact: with x = X 2^a
// (|X| < 2^11, x is FP16) and s = S 2^b (S < 2^24), any FP32 rounding
// boundary m = M 2^c (M odd, |M| < 2^25, c >= -150) differs from x / s by a
// nonzero multiple of 2^min(a, b + c) / (S 2^b), i.e. by more than
// min(2^(a-b-24), 2^(c-24)), while the double product is within
// 2^-51.9 |x / s| of x / s -- smaller than both terms whenever m is the
// boundary next to x / s.  x / s never equals a boundary exactly (the odd
// part of S M is at least 2^24 > |X|) except for a quotient below 2^-126,
// which needs |s| > 2^101: such threads divide in FP32 instead.
//
// INT8.  The clamp to [-128, 127] commutes with round-half-even, and adding
// 1.5 * 2^23 rounds to an integer (ties to even) whose two's-complement low
// byte is the code.
//
// FP8 e4m3fn.  After a clamp to +-448 (every value beyond 448 rounds there
// anyway) gfx950's v_cvt_pk_fp8_f32 rounds to the nearest OCP e4m3fn value,
// ties to even, subnormals included; the clamp makes its overflow mode
// irrelevant.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef _Float16 half_t;

// Tokens per thread: the thread issues the loads of all of them before it
// converts any, so each thread keeps kTokens x 16 bytes in flight (one load
// per thread leaves HBM idle behind the load latency).
#ifndef PKV_WRITE_TOKENS
#define PKV_WRITE_TOKENS 8
#endif
constexpr int kTokens = PKV_WRITE_TOKENS;

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(w >> 16));
}

// Eight FP32 quotients of one 16-byte chunk of FP16 values.
template <bool kDivide>
__device__ __forceinline__ void quotients(const uint4& raw, const float* s, const double* r,
                                          float* q) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float x = (k & 1) ? half_hi(w[k >> 1]) : half_lo(w[k >> 1]);
    if constexpr (kDivide)
      q[k] = x / s[k];  // IEEE division (correctly rounded)
    else
      q[k] = (float)((double)x * r[k]);
  }
}

// Codes of eight quotients, stored at dst.
template <int CT>
__device__ __forceinline__ void store_codes(const float* q, uint8_t* dst) {
  if constexpr (CT == PKV_F16) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = (uint32_t)__builtin_bit_cast(uint16_t, (half_t)q[2 * k]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (half_t)q[2 * k + 1]) << 16);
    *reinterpret_cast<uint4*>(dst) = uint4{o[0], o[1], o[2], o[3]};
  } else if constexpr (CT == PKV_I8) {
    uint32_t b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      b[k] = __float_as_uint(__builtin_amdgcn_fmed3f(q[k], -128.0f, 127.0f) + 12582912.0f);
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      o[h] = (b[4 * h] & 0xFFu) | ((b[4 * h + 1] & 0xFFu) << 8) | ((b[4 * h + 2] & 0xFFu) << 16) |
             (b[4 * h + 3] << 24);
    *reinterpret_cast<uint2*>(dst) = uint2{o[0], o[1]};
  } else {
    float c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_fmed3f(q[k], -448.0f, 448.0f);
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h], c[4 * h + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h + 2], c[4 * h + 3], v, true);
      o[h] = (uint32_t)v;
    }
    *reinterpret_cast<uint2*>(dst) = uint2{o[0], o[1]};
  }
}

template <int CT>
__global__ void __launch_bounds__(256) cache_write_kernel(const WriteArgs a) {
  // column = (KV head, 8-channel chunk of K then V) of a token row; the 1-D
  // index walks the columns of one group of kTokens tokens, then the next
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_head = a.chunks_k + a.chunks_v;
  const int64_t cols = (int64_t)a.kv_heads * per_head;
  const int64_t groups = ((int64_t)a.tokens + kTokens - 1) / kTokens;
  if (i >= groups * cols) return;
  int grp, col;
  if (groups * cols <= (int64_t)UINT32_MAX) {  // uniform: 32-bit division when it fits
    grp = (int)((uint32_t)i / (uint32_t)cols);
    col = (int)((uint32_t)i - (uint32_t)grp * (uint32_t)cols);
  } else {
    grp = (int)(i / cols);
    col = (int)(i - (int64_t)grp * cols);
  }
  const int g = col / per_head;
  int c = col - g * per_head;
  const bool is_k = c < a.chunks_k;
  if (!is_k) c -= a.chunks_k;
  const int dim = is_k ? a.head_size : a.v_head_size;
  const int d0 = 8 * c;
  const int quant = is_k ? a.k_quant : a.v_quant;
  const float* scale = is_k ? a.k_scale : a.v_scale;
  const uint16_t* src = (is_k ? a.key : a.value) + (size_t)g * dim + d0;
  const size_t src_stride = (size_t)a.kv_heads * dim;  // elements per token
  const int t0 = grp * kTokens;
  const int nt = min(kTokens, a.tokens - t0);

  // issue every load first: source chunks and slots of the group's tokens
  uint4 raw[kTokens];
  int64_t slot[kTokens];
#pragma unroll
  for (int j = 0; j < kTokens; ++j) {
    if (j < nt) {
      raw[j] = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + j) * src_stride);
      slot[j] = a.slot_mapping[t0 + j];
    } else {
      raw[j] = uint4{0u, 0u, 0u, 0u};
      slot[j] = -1;
    }
  }
  float s[8];
  if (quant == PKV_QUANT_PER_CHANNEL) {
    const float4 s0 = *reinterpret_cast<const float4*>(scale + (size_t)g * dim + d0);
    const float4 s1 = *reinterpret_cast<const float4*>(scale + (size_t)g * dim + d0 + 4);
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  } else {
    const float st = quant == PKV_QUANT_PER_TENSOR ? scale[0] : 1.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = st;
  }
  double r[8];
  bool divide = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    r[k] = 1.0 / (double)s[k];
    divide |= !(fabsf(s[k]) < 0x1p101f);
  }

  uint8_t* cache = is_k ? a.key_cache : a.value_cache;
  constexpr int kItem = CT == PKV_F16 ? 2 : 1;
  const size_t row_bytes = (size_t)a.kv_heads * dim * kItem;  // one slot
  uint8_t* dst0 = cache + ((size_t)g * dim + d0) * kItem;
#pragma unroll
  for (int j = 0; j < kTokens; ++j) {
    if (slot[j] < 0 || slot[j] >= a.n_slots) continue;  // not mapped (or past the group)
    float q[8];
    if (divide)
      quotients<true>(raw[j], s, r, q);
    else
      quotients<false>(raw[j], s, r, q);
    store_codes<CT>(q, dst0 + (size_t)slot[j] * row_bytes);
  }
}

hipError_t launch_cache_write(int cache_dtype, const WriteArgs& a, hipStream_t stream) {
  const int64_t groups = ((int64_t)a.tokens + kTokens - 1) / kTokens;
  const int64_t threads = groups * a.kv_heads * (a.chunks_k + a.chunks_v);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (cache_dtype) {
    case PKV_F16: hipLaunchKernelGGL(cache_write_kernel<PKV_F16>, grid, dim3(256), 0, stream, a); break;
    case PKV_I8: hipLaunchKernelGGL(cache_write_kernel<PKV_I8>, grid, dim3(256), 0, stream, a); break;
    case PKV_FP8_E4M3FN:
      hipLaunchKernelGGL(cache_write_kernel<PKV_FP8_E4M3FN>, grid, dim3(256), 0, stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
