// pkv_kernels.hip -- split-KV paged decode attention kernels for gfx950.
//
// Split kernel: one CTA per (split, KV head x 16-head block, row); four
// independent waves per CTA, each walking every fourth 16-token tile of the
// CTA's position range, with a one-tile register prefetch.  Per tile a wave
//   * gathers K and V rows through the block table (or a candidate list)
//     with 16-byte global loads straight into registers,
//   * converts INT8 / FP8-e4m3fn codes to FP16 exactly in registers (the
//     key scale is folded into the query once: Q' = fp16(Q * k_scale)),
//   * computes S^T = K Q'^T with v_mfma_f32_16x16x32_f16 (16 tokens x 16
//     heads; the GQA group is padded into the 16-wide N tile),
//   * runs the online softmax in FP32 with scores and running maximum in
//     natural-log units (only the difference is scaled by log2 e),
//   * accumulates O^T += V^T P^T with v_mfma_f32_16x16x16_f16, the FP16
//     probability tile taken directly from the score accumulator layout and
//     V^T built by in-register byte/half transposes of row segments.
// The four waves merge their (max, sum, accumulator) states through LDS in
// a fixed tree order and one partial per split is written: the accumulator
// times the value scale (applied once, after accumulation), the running
// maximum and the running sum.
//
// Combine kernel: one wave per (row, query head) merges the S partials in
// split order and applies the exact head-sink rescale 1 / (1 + exp(s_h - lse)).
//
// Sources on the pages: ONNX Runtime PR #33707 "Summary of Changes" sections
// 1-2 (Q' folding, value scale after accumulation, natural-log softmax, FP16
// probability tile, split-K partials and merge, candidate tiles with invalid
// entries); ONNX Runtime PR #29912 "Summary of Changes" (paged block-table
// decode with on-the-fly dequantisation, per-tensor / per-channel scales,
// LATENT layout, ApplyHeadSink, device-side lengths for graph safety);
// onnx-genai PR #1350 "Summary" (split count from static shapes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef _Float16 half_t;
typedef half_t half4 __attribute__((ext_vector_type(4)));
typedef half_t half8 __attribute__((ext_vector_type(8)));
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
// A wave rescales its accumulators only when a tile's maximum exceeds the
// running reference by more than this many nats, so probabilities stay
// below exp(8) ~ 2981, well inside FP16.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  // byte i of the result = byte sel.byte[i] of the 8-byte value {s0:s1}
  // (selectors 0-3 pick s1, 4-7 pick s0, 0x0C gives 0).
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// ---- exact code -> FP16 conversions (4 codes in a dword -> 4 halves) -------

// INT8: the binary16 pattern 0x6400 | u is 1024 + u for 0 <= u < 1024; with
// u = code + 128 (the code with its sign bit flipped) the value minus 1152 is
// the code, exactly.
__device__ __forceinline__ half4 i8x4_to_half4(uint32_t x) {
  const uint32_t u = x ^ 0x80808080u;
  const uint32_t lo = perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = perm(0x64646464u, u, 0x04030402u);
  half2_t a = __builtin_bit_cast(half2_t, lo);
  half2_t b = __builtin_bit_cast(half2_t, hi);
  const half2_t bias = {(half_t)-1152.0f, (half_t)-1152.0f};
  a = a + bias;
  b = b + bias;
  return half4{a[0], a[1], b[0], b[1]};
}

// FP8 e4m3fn (sign, 4 exponent bits with bias 7, 3 mantissa bits) moved bit
// for bit into binary16 (5 exponent bits, bias 15): the result is the code's
// value times 2^-8 for every finite code, normal or subnormal.  The 2^8 is
// folded into the score scale (K) and the value multiplier (V).
__device__ __forceinline__ uint32_t fp8x2_bits(uint32_t x, uint32_t sel) {
  const uint32_t p = perm(0u, x, sel);  // halves hold code << 8
  return ((p >> 1) & 0x3F803F80u) | (p & 0x80008000u);
}
__device__ __forceinline__ half4 fp8x4_to_half4(uint32_t x) {
  const uint32_t lo = fp8x2_bits(x, 0x010C000Cu);
  const uint32_t hi = fp8x2_bits(x, 0x030C020Cu);
  half2_t a = __builtin_bit_cast(half2_t, lo);
  half2_t b = __builtin_bit_cast(half2_t, hi);
  return half4{a[0], a[1], b[0], b[1]};
}

template <int CT>
__device__ __forceinline__ half4 codes4_to_half4(uint32_t x) {
  if constexpr (CT == PKV_I8) return i8x4_to_half4(x);
  else return fp8x4_to_half4(x);
}

// ---- global loads of NB bytes into dwords ---------------------------------

template <int NB>
__device__ __forceinline__ void load_bytes(const uint8_t* __restrict__ p, uint32_t* dst) {
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 16 * i);
      dst[4 * i + 0] = v.x;
      dst[4 * i + 1] = v.y;
      dst[4 * i + 2] = v.z;
      dst[4 * i + 3] = v.w;
    }
  } else if constexpr (NB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
    static_assert(NB == 4, "row segment of 4, 8 or a multiple of 16 bytes");
    dst[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// ---- the split kernel ---------------------------------------------------

template <int CT, int D, int VD, bool LATENT, bool GATHER>
struct SplitCfg {
  static constexpr int EB = (CT == PKV_F16) ? 2 : 1;   // bytes per code
  static constexpr int KROW = D * EB;                  // bytes of a K row
  static constexpr int VROW = VD * EB;                 // bytes of a V row
  static constexpr int NKS = D / 32;                   // QK k-steps (16x16x32)
  static constexpr int NKL = KROW / 64;                // 16-byte K loads per lane
  static constexpr int NKW = NKL * 4;                  // K dwords per lane
  static constexpr int VSEG = VROW / 16;               // V bytes per lane per row
  static constexpr int NVW = VSEG / 4;                 // V dwords per lane per row
  static constexpr int CPL = VD / 16;                  // channels per lane per row
  static constexpr int NCT = CPL;                      // PV col tiles
  static_assert(KROW % 64 == 0, "head_size * itemsize must be a multiple of 64");
  static_assert(VROW % 64 == 0, "v_head_size * itemsize must be a multiple of 64");
  static_assert(VD % 64 == 0, "v_head_size must be a multiple of 64");
};

template <class C>
struct Tile {
  uint32_t k[C::NKW];        // K row bytes of token (lane % 16)
  uint32_t v[4][C::NVW];     // V row segments of tokens 4j .. 4j+3
  uint32_t vmask;            // bit q: token 4j+q valid
};

template <int CT, int D, int VD, bool LATENT, bool GATHER>
__global__ void __launch_bounds__(kThreads)
split_kernel(const SplitArgs a) {
  using C = SplitCfg<CT, D, VD, LATENT, GATHER>;
  constexpr int W = kWaves;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;      // MFMA row/column index of this lane
  const int lj = lane >> 4;      // MFMA k-group of this lane

  const int split = blockIdx.x;
  const int g = blockIdx.y / a.head_blocks;
  const int hb = blockIdx.y - g * a.head_blocks;
  const int r = blockIdx.z;
  const int h0 = g * a.group + hb * 16;          // first query head of this CTA
  const int nh = min(16, a.group - hb * 16);     // query heads in this CTA
  const int S = a.num_splits;

  // ---- live extent of this split (device-side, graph safe) -------------
  const int cap = a.max_blocks_per_row * a.block_size;
  const int len = min(max(a.seq_lens[r], 0), cap);
  int npos = len;
  if constexpr (GATHER) npos = min(max(a.num_candidates[r], 0), a.max_candidates);
  const int n_act = npos > 0 ? min(S, (npos + a.min_chunk - 1) / a.min_chunk) : 0;
  const int chunk = n_act > 0 ? (((npos + n_act - 1) / n_act + 15) & ~15) : 0;
  const int p0 = split * chunk;
  const int p1 = min(npos, p0 + chunk);

  const size_t pair0 = (size_t)r * a.heads + h0;  // (row, first head) index
  if (split >= n_act || p0 >= npos) {
    // empty partial: m = -inf, l = 0 (the accumulator is never read)
    if (threadIdx.x < nh) {
      float2* ml = reinterpret_cast<float2*>(a.ws_ml) + (pair0 + threadIdx.x) * S + split;
      *ml = make_float2(kNegInf, 0.0f);
    }
    return;
  }

  // ---- Q' = fp16(Q * k_scale) as the B operand of the QK MFMA ------------
  // k-step ks, lane group lj holds channels d0(ks, lj) .. +7 of head li.
  half8 qop[C::NKS];
  {
    const bool hv = li < nh;
    const uint16_t* qrow = a.query + ((size_t)r * a.heads + h0 + (hv ? li : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      int d0;
      if constexpr (C::EB == 2) d0 = 32 * ks + 8 * lj;
      else d0 = 64 * (ks >> 1) + 16 * lj + 8 * (ks & 1);
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      const half8 q = __builtin_bit_cast(half8, raw);
      half8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float ks_e = 1.0f;
        if (a.k_quant == PKV_QUANT_PER_TENSOR) ks_e = a.k_scale[0];
        else if (a.k_quant == PKV_QUANT_PER_CHANNEL) ks_e = a.k_scale[(size_t)g * D + d0 + e];
        o[e] = hv ? (half_t)((float)q[e] * ks_e) : (half_t)0.0f;
      }
      qop[ks] = o;
    }
  }

  // ---- per-wave state -----------------------------------------------------
  f32x4 acc[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // running reference maximum of head li (natural log units)
  float l_part = 0.0f;     // this lane's share of the running sum

  const int ntiles = (p1 - p0 + 15) >> 4;
  const int64_t kv_stride_tok = (int64_t)a.kv_heads;  // rows per token slot
  const int32_t* bt_row = a.block_table + (size_t)r * a.max_blocks_per_row;

  // Issue the loads of tile t into `T` (addresses always inside the pool).
  auto issue = [&](Tile<C>& T, int t) {
    const int tp = p0 + 16 * t;  // first position of the tile
    int64_t slot_k;              // slot of token li
    int64_t slot_v[4];           // slots of tokens 4*lj + q
    bool valid_k;
    uint32_t vm = 0;
    if constexpr (!GATHER) {
      int blk = bt_row[tp / a.block_size];
      const bool bv = blk >= 0 && blk < a.num_pool_blocks;
      blk = bv ? blk : 0;
      const int64_t s0 = (int64_t)blk * a.block_size + (tp % a.block_size);
      slot_k = s0 + li;
      valid_k = bv && (tp + li < p1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        slot_v[q] = s0 + 4 * lj + q;
        vm |= (bv && (tp + 4 * lj + q < p1)) ? (1u << q) : 0u;
      }
    } else {
      const int pos = tp + li;
      int c = pos < p1 ? a.candidates[(size_t)r * a.max_candidates + pos] : -1;
      bool v = c >= 0 && c < len;
      int blk = v ? bt_row[c / a.block_size] : 0;
      v = v && blk >= 0 && blk < a.num_pool_blocks;
      const int64_t s = v ? (int64_t)blk * a.block_size + (c % a.block_size) : 0;
      slot_k = s;
      valid_k = v;
      const int vi = v ? 1 : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int src = 4 * lj + q;
        const int lo = __shfl((int)(s & 0xffffffff), src);
        const int hi = __shfl((int)(s >> 32), src);
        slot_v[q] = ((int64_t)hi << 32) | (uint32_t)lo;
        vm |= __shfl(vi, src) ? (1u << q) : 0u;
      }
    }
    (void)valid_k;
    // K: bytes [64 s + 16 lj, +16) of token li's row, s = 0 .. NKL-1
    const uint8_t* krow = a.key_cache + ((size_t)slot_k * kv_stride_tok + g) * C::KROW;
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) load_bytes<16>(krow + 64 * s + 16 * lj, &T.k[4 * s]);
    // V: bytes [li * VSEG, +VSEG) of the rows of tokens 4 lj + q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint8_t* vrow;
      if constexpr (LATENT) vrow = a.key_cache + ((size_t)slot_v[q] * kv_stride_tok + g) * C::KROW;
      else vrow = a.value_cache + ((size_t)slot_v[q] * kv_stride_tok + g) * C::VROW;
      load_bytes<C::VSEG>(vrow + li * C::VSEG, T.v[q]);
    }
    T.vmask = vm;
  };

  // Consume tile T: scores, online softmax, PV.
  auto consume = [&](const Tile<C>& T) {
    // S^T = K Q'^T : lane holds scores of tokens 4 lj + q for head li
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) {
      if constexpr (C::EB == 2) {
        const half8 kop = __builtin_bit_cast(
            half8, uint4{T.k[4 * s], T.k[4 * s + 1], T.k[4 * s + 2], T.k[4 * s + 3]});
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[s], sacc, 0, 0, 0);
      } else {
        const half4 c0 = codes4_to_half4<CT>(T.k[4 * s + 0]);
        const half4 c1 = codes4_to_half4<CT>(T.k[4 * s + 1]);
        const half4 c2 = codes4_to_half4<CT>(T.k[4 * s + 2]);
        const half4 c3 = codes4_to_half4<CT>(T.k[4 * s + 3]);
        const half8 k0 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const half8 k1 = {c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qop[2 * s], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qop[2 * s + 1], sacc, 0, 0, 0);
      }
    }
    float sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sc[q] = ((T.vmask >> q) & 1u) ? sacc[q] * a.score_scale : kNegInf;
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_ref + kRescaleSlack;
    if (__any(need)) {
      const float mn = fmaxf(m_ref, mt);
      const float alpha = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - mn) * kLog2e);
      l_part *= alpha;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) acc[ct] *= alpha;
      m_ref = mn;
    }
    const float mu = (m_ref == kNegInf) ? 0.0f : m_ref;
    float p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = __builtin_amdgcn_exp2f((sc[q] - mu) * kLog2e);
    l_part += (p[0] + p[1]) + (p[2] + p[3]);
    const half4 pop = {(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3]};

    // V^T operands: for col tile ct, lane holds channel li*CPL+ct of tokens
    // 4 lj .. 4 lj + 3 (rows q = 0..3 of its segments), transposed in registers
    uint32_t vz[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vz[q] = ((T.vmask >> q) & 1u) ? 0xffffffffu : 0u;
    if constexpr (C::EB == 2) {
#pragma unroll
      for (int w = 0; w < C::NVW; ++w) {
        const uint32_t r0 = T.v[0][w] & vz[0], r1 = T.v[1][w] & vz[1];
        const uint32_t r2 = T.v[2][w] & vz[2], r3 = T.v[3][w] & vz[3];
        // channel 2w: low halves; channel 2w+1: high halves
        const uint32_t a01 = perm(r1, r0, 0x05040100u), a23 = perm(r3, r2, 0x05040100u);
        const uint32_t b01 = perm(r1, r0, 0x07060302u), b23 = perm(r3, r2, 0x07060302u);
        const half4 va = __builtin_bit_cast(half4, uint2{a01, a23});
        const half4 vb = __builtin_bit_cast(half4, uint2{b01, b23});
        acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pop, acc[2 * w], 0, 0, 0);
        acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vb, pop, acc[2 * w + 1], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int w = 0; w < C::NVW; ++w) {
        const uint32_t r0 = T.v[0][w] & vz[0], r1 = T.v[1][w] & vz[1];
        const uint32_t r2 = T.v[2][w] & vz[2], r3 = T.v[3][w] & vz[3];
        const uint32_t t0 = perm(r1, r0, 0x05010400u), t1 = perm(r1, r0, 0x07030602u);
        const uint32_t t2 = perm(r3, r2, 0x05010400u), t3 = perm(r3, r2, 0x07030602u);
        const uint32_t o0 = perm(t2, t0, 0x05040100u), o1 = perm(t2, t0, 0x07060302u);
        const uint32_t o2 = perm(t3, t1, 0x05040100u), o3 = perm(t3, t1, 0x07060302u);
        acc[4 * w + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_half4<CT>(o0), pop, acc[4 * w + 0], 0, 0, 0);
        acc[4 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_half4<CT>(o1), pop, acc[4 * w + 1], 0, 0, 0);
        acc[4 * w + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_half4<CT>(o2), pop, acc[4 * w + 2], 0, 0, 0);
        acc[4 * w + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_half4<CT>(o3), pop, acc[4 * w + 3], 0, 0, 0);
      }
    }
  };

  // ---- main loop: wave `wave` takes tiles wave, wave + W, ... -------------
  {
    Tile<C> A, B;
    int t = wave;
    if (t < ntiles) issue(A, t);
    while (t < ntiles) {
      if (t + W < ntiles) issue(B, t + W);
      consume(A);
      t += W;
      if (t >= ntiles) break;
      if (t + W < ntiles) issue(A, t + W);
      consume(B);
      t += W;
    }
  }

  // ---- merge the W wave states (fixed order) and publish the partial -----
  // l: sum the four lane groups of head li
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);

  __shared__ float sm_m[W][16];
  __shared__ float sm_l[W][16];
  constexpr int NACC = C::NCT * 4;                 // accumulator floats per lane
  __shared__ float sm_acc[(W / 2) * NACC * 64];    // [slot][element][lane]

  if (lane < 16) {
    sm_m[wave][lane] = m_ref;
    sm_l[wave][lane] = l_part;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][li]);
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float mw = sm_m[w][li];
    const float f = (mw == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((mw - M) * kLog2e);
    L += f * sm_l[w][li];
  }
  {
    const float f = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - M) * kLog2e);
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) acc[ct] *= f;
  }
#pragma unroll
  for (int half = W / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      float* dst = sm_acc + (size_t)(wave - half) * NACC * 64;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[(ct * 4 + q) * 64 + lane] = acc[ct][q];
    }
    __syncthreads();
    if (wave < half) {
      const float* src = sm_acc + (size_t)wave * NACC * 64;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ct][q] += src[(ct * 4 + q) * 64 + lane];
    }
    __syncthreads();
  }

  if (wave == 0 && li < nh) {
    const int h = h0 + li;
    const size_t pidx = ((size_t)r * a.heads + h) * S + split;
    if (lj == 0) reinterpret_cast<float2*>(a.ws_ml)[pidx] = make_float2(M, L);
    // lane holds channels (4 lj + q) * CPL + ct; write them with the value
    // scale applied once.
    float* dst = a.ws_acc + pidx * VD;
    const float* vs = a.v_scale;
    const int vstride = a.v_scale_stride;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cbase = (4 * lj + q) * C::CPL;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ct += 4) {
        float4 o;
        float* op = reinterpret_cast<float*>(&o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float vsc = 1.0f;
          if (a.v_quant == PKV_QUANT_PER_TENSOR) vsc = vs[0];
          else if (a.v_quant == PKV_QUANT_PER_CHANNEL) vsc = vs[(size_t)g * vstride + cbase + ct + e];
          op[e] = (acc[ct + e][q] * a.v_mult) * vsc;
        }
        *reinterpret_cast<float4*>(dst + cbase + ct) = o;
      }
    }
  }
}

// ---- the combine kernel ---------------------------------------------------

constexpr int kCombineWaves = 4;

template <int VD, bool OUT_F32>
__global__ void __launch_bounds__(64 * kCombineWaves)
combine_kernel(const CombineArgs a) {
  constexpr int CPT = VD / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (pair >= a.rows * a.heads) return;
  const int h = pair % a.heads;
  const int S = a.num_splits;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (size_t)pair * S;

  float mk = kNegInf, lk = 0.0f;
  if (lane < S) {
    const float2 v = ml[lane];
    mk = v.x;
    lk = v.y;
  }
  float M = mk;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float w = (mk == kNegInf) ? 0.0f : expf(mk - M);
  float L = w * lk;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);

  float o[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) o[e] = 0.0f;
  const float* accp = a.ws_acc + (size_t)pair * S * VD + lane * CPT;
  for (int k = 0; k < S; ++k) {
    const float wk = __shfl(w, k);
    if (wk != 0.0f) {  // uniform: empty splits' accumulators are never read
      const float* src = accp + (size_t)k * VD;
      if constexpr (CPT >= 4) {
#pragma unroll
        for (int e = 0; e < CPT; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + e);
          o[e] += wk * v.x;
          o[e + 1] += wk * v.y;
          o[e + 2] += wk * v.z;
          o[e + 3] += wk * v.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < CPT; ++e) o[e] += wk * src[e];
      }
    }
  }

  float lse = kNegInf;
  float f = 0.0f;
  if (L > 0.0f) {
    lse = M + logf(L);
    f = 1.0f / L;
    if (a.head_sink) f *= 1.0f / (1.0f + expf(a.head_sink[h] - lse));
  }
  if (a.lse_out && lane == 0) a.lse_out[pair] = lse;
  if constexpr (OUT_F32) {
    float* dst = reinterpret_cast<float*>(a.out) + (size_t)pair * VD + lane * CPT;
#pragma unroll
    for (int e = 0; e < CPT; ++e) dst[e] = o[e] * f;
  } else {
    half_t* dst = reinterpret_cast<half_t*>(a.out) + (size_t)pair * VD + lane * CPT;
#pragma unroll
    for (int e = 0; e < CPT; ++e) dst[e] = (half_t)(o[e] * f);
  }
}

// ---- dispatch ---------------------------------------------------------------

template <int CT, int D, int VD, bool LAT, bool GA>
static hipError_t launch_one(const SplitArgs& a, hipStream_t stream) {
  dim3 grid(a.num_splits, a.kv_heads * a.head_blocks, a.rows);
  hipLaunchKernelGGL((split_kernel<CT, D, VD, LAT, GA>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int CT, int D, int VD, bool LAT, bool GA>
static hipError_t occupancy_one(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, split_kernel<CT, D, VD, LAT, GA>,
                                                       kThreads, 0);
}

// Calls F<CT, D, VD, LAT, GA>(args...) for the compiled variant; returns
// hipErrorInvalidValue for a variant that is not compiled.
#define PKV_FOR_VARIANT(v, CALL)                                                   \
  do {                                                                             \
    const int hs = (v).head_size, vhs = (v).v_head_size;                           \
    const bool lat = (v).latent != 0, ga = (v).gathered != 0;                      \
    switch ((v).cache_dtype) {                                                     \
      case PKV_F16: PKV_SHAPES(PKV_F16, CALL); break;                              \
      case PKV_I8: PKV_SHAPES(PKV_I8, CALL); break;                                \
      case PKV_FP8_E4M3FN: PKV_SHAPES(PKV_FP8_E4M3FN, CALL); break;                \
      default: break;                                                              \
    }                                                                              \
  } while (0)

#define PKV_GATHER(CT, D, VD, LAT, CALL) \
  do { if (ga) { CALL(CT, D, VD, LAT, true); } else { CALL(CT, D, VD, LAT, false); } } while (0)

#define PKV_SHAPES(CT, CALL)                                                       \
  do {                                                                             \
    if (!lat && hs == 64 && vhs == 64) PKV_GATHER(CT, 64, 64, false, CALL);        \
    else if (!lat && hs == 128 && vhs == 128) PKV_GATHER(CT, 128, 128, false, CALL);\
    else if (!lat && hs == 256 && vhs == 256) PKV_GATHER(CT, 256, 256, false, CALL);\
    else if (lat && hs == 576 && vhs == 512) PKV_GATHER(CT, 576, 512, true, CALL); \
  } while (0)

bool variant_supported(const Variant& v) {
  bool ok = false;
#define PKV_MARK(CT, D, VD, LAT, GA) ok = true
  PKV_FOR_VARIANT(v, PKV_MARK);
#undef PKV_MARK
  return ok;
}

hipError_t launch_split(const Variant& v, const SplitArgs& a, hipStream_t stream) {
  hipError_t err = hipErrorInvalidValue;
#define PKV_LAUNCH(CT, D, VD, LAT, GA) err = launch_one<CT, D, VD, LAT, GA>(a, stream)
  PKV_FOR_VARIANT(v, PKV_LAUNCH);
#undef PKV_LAUNCH
  return err;
}

hipError_t split_occupancy(const Variant& v, int* ctas_per_cu) {
  hipError_t err = hipErrorInvalidValue;
#define PKV_OCC(CT, D, VD, LAT, GA) err = occupancy_one<CT, D, VD, LAT, GA>(ctas_per_cu)
  PKV_FOR_VARIANT(v, PKV_OCC);
#undef PKV_OCC
  return err;
}

template <int VD, bool F32>
static hipError_t launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  const int pairs = a.rows * a.heads;
  const int blocks = (pairs + kCombineWaves - 1) / kCombineWaves;
  hipLaunchKernelGGL((combine_kernel<VD, F32>), dim3(blocks), dim3(64 * kCombineWaves), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_combine(int v_head_size, int out_dtype, const CombineArgs& a,
                          hipStream_t stream) {
  const bool f32 = out_dtype == PKV_F32;
  switch (v_head_size) {
    case 64: return f32 ? launch_combine_t<64, true>(a, stream) : launch_combine_t<64, false>(a, stream);
    case 128: return f32 ? launch_combine_t<128, true>(a, stream) : launch_combine_t<128, false>(a, stream);
    case 256: return f32 ? launch_combine_t<256, true>(a, stream) : launch_combine_t<256, false>(a, stream);
    case 512: return f32 ? launch_combine_t<512, true>(a, stream) : launch_combine_t<512, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
