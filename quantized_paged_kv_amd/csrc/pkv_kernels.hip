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
// Combine kernel: one CTA per (row, query head) merges the S partials in a
// fixed order and applies the exact head-sink rescale 1 / (1 + exp(s_h - lse)).
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

#include <type_traits>

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

// FP8 e4m3fn: gfx950 converts two OCP e4m3fn codes to two FP16 values per
// instruction; every finite code is exactly representable in FP16 (verified
// on the device for all 256 codes; NaN codes stay NaN and are outside the
// cache's domain).
__device__ __forceinline__ half4 fp8x4_to_half4(uint32_t x) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  return half4{a[0], a[1], b[0], b[1]};
}

template <int CT>
__device__ __forceinline__ half4 codes4_to_half4(uint32_t x) {
  if constexpr (CT == PKV_I8) return i8x4_to_half4(x);
  else return fp8x4_to_half4(x);
}

// ---- robust numerics --------------------------------------------------------
//
// The fast path rounds two things to FP16: the folded query Q' = Q k_scale
// and the probability tile P.  Following the INT8 DynamicSparseAttention
// page (ONNX Runtime PR #33707, "Numerics": the table of review cases and
// the follow-up review thread), each CTA guards both:
//   * P enters the PV products as FP16(16 p) and, when the values are large
//     enough for its rounding to matter, also as the FP16 residual (a second
//     MFMA), so a probability keeps about 22 bits and values of opposite
//     sign do not cancel through rounding; the factor 16 is exact and
//     removed with the value scale (p <= e^8, the rescale slack, so 16 p
//     stays below FP16's maximum);
//   * the folding error of Q' is bounded per head,
//       eps_h = scale * sum_d |fp16(Q_d ks_d) - Q_d ks_d| * max|code|,
//     and a CTA with eps_h above 0.125 nats recomputes its partial on an
//     FP32 path;
//   * with quantised values, a CTA whose tile held a probability below
//     FP16's normal range (16 p < 2^-14) recomputes on the FP32 path when
//     max|value_scale| * max|code| * tokens >= 2^17, i.e. when such
//     probabilities can move the output by more than about 2^-12.
// The FP32 path evaluates the definition directly: unfolded Q k_scale in
// FP32, exact running maximum in natural-log units, FP32 sums, and the value
// scale applied after accumulation.
constexpr float kProbScale = 16.0f;
constexpr float kFoldBudget = 0.125f;          // nats
constexpr float kTailLog = -12.47664925f;      // ln(2^-18): 16 p below 2^-14
constexpr float kTailArm = 131072.0f;          // 2^17
#ifndef PKV_RESIDUAL_TILE
#define PKV_RESIDUAL_TILE 1
#endif
constexpr bool kResidualTile = PKV_RESIDUAL_TILE != 0;

// largest |code| of a cache format (FP16: the largest finite value)
template <int CT>
__device__ __forceinline__ float code_bound() {
  if constexpr (CT == PKV_I8) return 128.0f;
  else if constexpr (CT == PKV_FP8_E4M3FN) return 448.0f;
  else return 65504.0f;
}

// FP16(16 p) and, with LO, the FP16 residual of that rounding
template <bool LO>
__device__ __forceinline__ void split_prob(const float (&p)[4], half4& hi, half4& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float ps = p[q] * kProbScale;
    hi[q] = (half_t)ps;
    if constexpr (LO) lo[q] = (half_t)(ps - (float)hi[q]);
  }
}

// exact value of the code at byte offset `i` of a row (FP16: element i)
template <int CT>
__device__ __forceinline__ float code_at(const uint8_t* row, int i) {
  if constexpr (CT == PKV_F16) {
    return (float)reinterpret_cast<const half_t*>(row)[i];
  } else if constexpr (CT == PKV_I8) {
    return (float)reinterpret_cast<const int8_t*>(row)[i];
  } else {
    return (float)__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)row[i], 1.0f, false)[0];
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// ---- wave-uniform reads ----------------------------------------------------
//
// A value every lane of a wave needs at the same index (a block id of a
// 16-token tile, a row length) is read with a scalar load through the
// constant address space: it lands in an SGPR and is waited for with the
// scalar/LDS counter.  Read as a vector load, waiting for it would also wait
// for every K/V load issued before it (vector loads complete in order),
// draining the prefetch pipeline.  The arrays read this way (block table,
// lengths) are never written while a kernel runs.
typedef const __attribute__((address_space(4))) int32_t cint32_t;

__device__ __forceinline__ int uniform_load(const int32_t* p, size_t idx) {
  return ((cint32_t*)p)[idx];  // address-space cast (C-style; not expressible as a C++ cast)
}

__device__ __forceinline__ float uniform_load(const float* p, size_t idx) {
  return ((const __attribute__((address_space(4))) float*)p)[idx];
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
  // Prefetch depth (tiles held in registers per wave: one consumed, the rest
  // in flight) and the register budget (waves per SIMD), chosen by
  // measurement on MI355X: for head sizes up to 128 three waves per SIMD
  // beat two; and one tile in flight (two for the smallest tiles) beat two
  // (three): more outstanding loads per CU only lengthen their latency (the
  // single-row INT8 head-256 step 7.35 -> 6.75 us, the gathered one 10.9
  // -> 9.6, the 64-row one 59.3 -> 58.6).
  static constexpr int TILE_REGS = NKW + 4 * NVW;
  static constexpr int NST = TILE_REGS <= 16 ? 3 : 2;
  static constexpr int MIN_WAVES =
      LATENT ? 1 : (TILE_REGS <= 32 && VD <= 128 && !GATHER ? 3 : (TILE_REGS <= 40 ? 2 : 1));
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

constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit dword format (gfx9)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// Direct-to-LDS loads (gfx950 `buffer_load_dwordx4 ... lds`): lane i's 16
// bytes land at LDS address m0 + 16 i, nothing passes through registers,
// and offsets past the descriptor's size land as zeros.  Written as inline
// assembly because the compiler, seeing such a load, makes every later LDS
// read wait for all outstanding vector loads (which would drain the
// prefetch); the kernel therefore waits for them itself, with vmcnt counts
// that follow its own issue order (wait_vmcnt).  The descriptor is the
// same raw-buffer one as make_rsrc's, as four SGPRs.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, (uint32_t)kBufferWord3};
}

__device__ __forceinline__ void buffer_load_lds16(uint32_t lds, uint32_t voff, u32x4 rsrc) {
  // the LDS address goes in through m0 as an input operand, so the compiler
  // sets m0 itself and knows what it holds
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// wait until at most N vector memory operations of this wave are
// outstanding (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// 16 / 8 / 4 bytes from a buffer; offsets past the descriptor's size read 0
// without a memory request.
template <int NB>
__device__ __forceinline__ void buffer_bytes(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                             uint32_t soff, uint32_t* dst) {
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, 0);
      const uint4 u = __builtin_bit_cast(uint4, v);
      dst[4 * i + 0] = u.x;
      dst[4 * i + 1] = u.y;
      dst[4 * i + 2] = u.z;
      dst[4 * i + 3] = u.w;
    }
  } else if constexpr (NB == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    const uint2 u = __builtin_bit_cast(uint2, v);
    dst[0] = u.x;
    dst[1] = u.y;
  } else {
    static_assert(NB == 4, "row segment of 4, 8 or a multiple of 16 bytes");
    dst[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
  }
}

// Live positions of row i: clamped context length (dense rows) or clamped
// candidate-list length (gathered rows).
template <bool GATHER>
__device__ __forceinline__ int row_positions(const SplitArgs& a, int i, int cap) {
  if constexpr (GATHER) return min(max(a.num_candidates[i], 0), a.max_candidates);
  else return min(max(a.seq_lens[i], 0), cap);
}

// The work item (row, unit = KV head x 16-head block, split) a CTA runs.
struct Work {
  int r, u, split, n_row, npos, len;
  int g, hb, h0, nh;  // KV head, head block, first query head, query heads (<= 16)
  // Sliding window: the row attends tokens [lo, len).  Dense rows number
  // their positions from base = lo rounded down to a multiple of 16 (token =
  // base + position, so tiles never straddle a block); positions before
  // lo - base are masked.  Without a window lo = base = 0.
  int lo, base;
};

// The kernels are instantiated twice: EXT = false for problems without a
// sliding window or soft cap (none of the code below is compiled in), and
// EXT = true for the rest.

// First token of a row's sliding window (0 without one).  With T query
// tokens per row, token j's window ends at len - (T - 1 - j), so the row's
// range starts at the first token's window start (each later token's own
// start is masked per head slot).
template <bool EXT>
__device__ __forceinline__ int window_lo(const SplitArgs& a, int len) {
  if constexpr (!EXT) return 0;
  const int first = len - (a.qtok - 1);  // positions the row's first token attends
  return (a.window > 0 && first > a.window) ? first - a.window : 0;
}

// Logit soft cap x -> c tanh(x / c) (identity without one).
template <bool EXT>
__device__ __forceinline__ float soft_cap(const SplitArgs& a, float x) {
  if constexpr (!EXT) return x;
  return a.softcap > 0.0f ? a.softcap * tanhf(x * a.inv_softcap) : x;
}

// Scaled (and capped) scores of a 4-token MFMA column; the cap is one
// uniform branch around all four, taken before the masking select.
template <bool EXT>
__device__ __forceinline__ void scaled_scores(const SplitArgs& a, const f32x4& acc, float (&x)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) x[q] = acc[q] * a.score_scale;
  if constexpr (EXT) {
    if (a.softcap > 0.0f) {
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = a.softcap * tanhf(x[q] * a.inv_softcap);
    }
  }
}

// Locate this CTA's work item (device-side, graph safe).  Returns false for
// a padding CTA past the last item.
// Live-balanced mode (target_ctas > 0): one chunk length c for every row,
// from the total live positions of all rows and the CTAs aimed at; row r
// gets n_r = clamp(ceil(npos_r / c), 1, S) splits, and the work items
// (row, unit, split) are numbered row by row, so consecutive CTAs -- which
// the hardware spreads round-robin over the XCDs -- carry equal work and no
// CTA launches only to find nothing to do (except trailing padding).  All
// row lengths are read in one round trip (lane i holds rows i + 64 k,
// k < NR; the loads are issued unconditionally, from clamped indices).
// locate_balanced takes NR = 1 for up to 64 rows, the common decode batch
// (C3-shaped steps 0.4 us faster than reading NR = 16 lengths per lane).
template <bool GATHER, bool EXT, int NR>
__device__ __forceinline__ bool locate_rows(const SplitArgs& a, int lane, Work& w) {
  const int S = a.num_splits;
  const int units_row = a.units_row;
  const int cap = a.max_blocks_per_row * a.block_size;
  const int c = blockIdx.x;
  int raw[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int rr = min(lane + 64 * i, a.rows - 1);
    raw[i] = GATHER ? a.num_candidates[rr] : a.seq_lens[rr];
  }
  int np[NR];
  // (the host uses this decomposition only when rows * capacity < 2^31, so
  // the total fits 32 bits)
  int tot = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int rr = lane + 64 * i;
    np[i] = rr < a.rows ? min(max(raw[i], 0), GATHER ? a.max_candidates : cap) : 0;
  }
  // dense rows with a sliding window: positions from the window start
  // rounded down to 16 (one uniform branch; np holds the clamped lengths)
  if constexpr (!GATHER && EXT)
    if (a.window > 0) {
#pragma unroll
      for (int i = 0; i < NR; ++i) np[i] -= window_lo<EXT>(a, np[i]) & ~15;
    }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    tot += np[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  const int64_t work = (int64_t)__builtin_amdgcn_readfirstlane(tot) * units_row;
  const int64_t cl = (work + a.target_ctas - 1) / a.target_ctas;
  const int cgl = max(a.min_chunk, (int)min<int64_t>(((cl + 15) >> 4) << 4, 1 << 30));
  int base = 0;
  int r = -1, u = 0, split = 0, n_row = 0, npos = 0, rlen = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (64 * i >= a.rows) break;
    const int rr = lane + 64 * i;
    // (capacities are at most 2^30 positions, so nothing here overflows)
    const int n = rr < a.rows ? min(S, max(1, (np[i] + cgl - 1) / cgl)) : 0;
    const int items = n * units_row;
    int incl = items;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int excl = incl - items;
    const bool hit = c >= base + excl && c < base + incl;
    const uint64_t m = __ballot(hit);
    if (m) {
      const int src = __builtin_ctzll(m);
      r = 64 * i + src;
      const int off = c - base - __shfl(excl, src);
      n_row = __shfl(n, src);
      npos = __shfl(np[i], src);
      if constexpr (!GATHER && EXT) rlen = min(max(__shfl(raw[i], src), 0), cap);
      u = off / n_row;
      split = off - u * n_row;
      break;
    }
    base += __shfl(incl, 63);
  }
  r = __builtin_amdgcn_readfirstlane(r);
  if (r < 0) return false;
  w.r = r;
  w.u = __builtin_amdgcn_readfirstlane(u);
  w.split = __builtin_amdgcn_readfirstlane(split);
  w.n_row = __builtin_amdgcn_readfirstlane(n_row);
  w.npos = __builtin_amdgcn_readfirstlane(npos);
  // dense rows: the clamped length (npos without a window); gathered rows
  // get theirs in finish_item
  w.len = (!GATHER && EXT) ? __builtin_amdgcn_readfirstlane(rlen) : w.npos;
  w.lo = GATHER ? 0 : window_lo<EXT>(a, w.len);
  w.base = GATHER ? 0 : (w.lo & ~15);
  return true;
}

template <bool GATHER, bool EXT>
__device__ __forceinline__ bool locate_balanced(const SplitArgs& a, int lane, Work& w) {
  if (a.rows <= 64) return locate_rows<GATHER, EXT, 1>(a, lane, w);
  return locate_rows<GATHER, EXT, kMaxBalancedRows / 64>(a, lane, w);
}

// Static mode (target_ctas == 0): CTA c is item c of the (row, unit,
// split < S) list; nothing is read.
__device__ __forceinline__ void static_item(const SplitArgs& a, Work& w) {
  const int S = a.num_splits;
  const int units_row = a.units_row;
  const int c = blockIdx.x;
  w.r = c / (units_row * S);
  const int rem = c - w.r * units_row * S;
  w.u = rem / S;
  w.split = rem - w.u * S;
  w.n_row = S;
  w.npos = w.len = 0;
  w.lo = w.base = 0;
}

// Several query tokens per row (MT, the multi-token decode of speculative
// and chunked steps): the T tokens of a row share its block-table row and
// attend causally, token j the positions [0, len - T + 1 + j).  The (token,
// query head) pairs of one KV head are its "virtual heads" v = j * group + h
// (T * group of them), taken 16 per head block like the query heads of one
// token, so every KV tile a CTA reads serves all the tokens of its heads.
template <bool MT = false>
__device__ __forceinline__ void unit_heads(const SplitArgs& a, Work& w) {
  w.g = w.u / a.head_blocks;
  w.hb = w.u - w.g * a.head_blocks;
  if constexpr (MT) {
    w.h0 = w.g * a.group;
    w.nh = min(16, a.qtok * a.group - w.hb * 16);
  } else {
    w.h0 = w.g * a.group + w.hb * 16;
    w.nh = min(16, a.group - w.hb * 16);
  }
}

// Head slot e (0 <= e < w.nh) of a work unit: its (row, query token, head)
// as the index of the query / output / lse row, the query head, and the
// token.  One token per row: head h0 + e of row r.  Several: virtual head
// hb * 16 + e of the unit's KV heads g, g + 1, ... (T * group each; units
// of several KV heads have one head block).
struct HeadSlot {
  size_t pair;  // (row * T + token) * heads + head
  int h;        // query head
  int tok;      // query token of the row
};

template <bool MT = false>
__device__ __forceinline__ HeadSlot head_slot(const SplitArgs& a, const Work& w, int e) {
  if constexpr (!MT) {
    return HeadSlot{(size_t)w.r * a.heads + w.h0 + e, w.h0 + e, 0};
  } else {
    const int vg = a.qtok * a.group;  // virtual heads per KV head
    const int va = w.hb * 16 + e;
    const int go = va / vg;           // KV head g + go
    const int v = va - go * vg;
    const int j = v / a.group;
    const int h = (w.g + go) * a.group + (v - j * a.group);
    return HeadSlot{((size_t)w.r * a.qtok + j) * a.heads + h, h, j};
  }
}

// Clamped lengths from the raw values read in the prologue: raw_npos (static
// mode: seq_len, or num_candidates of gathered rows) and raw_len (gathered
// rows: seq_len, which bounds the valid candidate indices).
template <bool GATHER, bool EXT>
__device__ __forceinline__ void finish_item(const SplitArgs& a, Work& w, bool balanced,
                                            int raw_npos, int raw_len) {
  const int cap = a.max_blocks_per_row * a.block_size;
  if constexpr (GATHER) {
    if (!balanced) w.npos = min(max(raw_npos, 0), a.max_candidates);
    w.len = min(max(raw_len, 0), cap);
    w.lo = window_lo<EXT>(a, w.len);
    w.base = 0;
  } else {
    if (!balanced) w.len = min(max(raw_npos, 0), cap);
    w.lo = window_lo<EXT>(a, w.len);
    w.base = w.lo & ~15;
    w.npos = w.len - w.base;
  }
}

// Position range [p0, p1) of the work item; publishes the empty partials
// (m = -inf, l = 0; accumulators are never read) this CTA is responsible
// for and returns false when its own range is empty.  Live-balanced mode:
// the row's n_row splits share its positions evenly in 16-position steps.
// Static mode: split k covers [k c, (k + 1) c) with the host's chunk c, so
// p0 is known before any length is read.
__device__ __forceinline__ int static_p0(const SplitArgs& a, int split) {
  return split * a.static_chunk;
}

// ---- direct output (one split per row) -------------------------------------
//
// With S = 1 the combine would take the single partial unchanged: M = m,
// L = 1 * l, O = (0 + 1 * partial) / L, lse = M + log L, then the head sink.
// The split kernel does exactly these operations itself (same order, so
// the result is bitwise the combine's) and writes the output.
struct Final {
  float f;    // factor applied to the partial (0 for an empty row)
  float lse;
};

__device__ __forceinline__ Final final_of(const SplitArgs& a, int h, float M, float L) {
  Final r{0.0f, kNegInf};
  if (L > 0.0f) {
    r.lse = M + logf(L);
    r.f = 1.0f / L;
    if (a.head_sink) r.f *= 1.0f / (1.0f + expf(a.head_sink[h] - r.lse));
  }
  return r;
}

// Four output channels c .. c+3 of (row, head) pair `pair` from partial values.
template <int VD>
__device__ __forceinline__ void store_final(const SplitArgs& a, size_t pair, int c, float4 part,
                                            float f) {
  const float4 r = make_float4(0.0f + part.x, 0.0f + part.y, 0.0f + part.z, 0.0f + part.w);
  if (a.out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + pair * VD + c) =
        make_float4(r.x * f, r.y * f, r.z * f, r.w * f);
  } else {
    const half4 hv = {(half_t)(r.x * f), (half_t)(r.y * f), (half_t)(r.z * f), (half_t)(r.w * f)};
    *reinterpret_cast<half4*>(reinterpret_cast<half_t*>(a.out) + pair * VD + c) = hv;
  }
}

// Added to a buffer offset, puts the access past any descriptor's range, so
// the load returns zeros without a memory request.
constexpr uint32_t kPastDescriptor = 0x40000000u;

// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt not waited.
constexpr int kWaitVmcnt0 = 0x0F70;

// First position of the work item's range (the p0 split_range computes);
// known before any row length is read in the static mode.
__device__ __forceinline__ int split_p0(const SplitArgs& a, const Work& w) {
  if (a.target_ctas > 0)
    return w.n_row > 0 ? w.split * (((w.npos + w.n_row - 1) / w.n_row + 15) & ~15) : 0;
  return static_p0(a, w.split);
}

// Block ids of one wave's tiles (dense rows).  The wave takes tiles
// wave + W k; lane k of one VGPR holds the block of the wave's tile
// 64 win + k, read with one vector load per 64 tiles and picked per tile
// with readlane, so the tile loop has no dependent memory read (a scalar
// load that misses would wait behind the streaming K/V traffic).
struct WaveBlocks {
  const int32_t* bt_row;
  int p0, wave, nw, win, ids;  // p0: token of the wave's tile 0 position; nw: waves of the CTA

  __device__ __forceinline__ void load(const SplitArgs& a, int w_idx, int lane) {
    win = w_idx;
    const int t = wave + nw * (64 * w_idx + lane);
    const int bi = min(max((p0 + 16 * t) >> a.log2_block, 0), a.max_blocks_per_row - 1);
    ids = bt_row[bi];
  }
  // block id of the wave's tile t (t = wave + W k)
  __device__ __forceinline__ int of(const SplitArgs& a, int t, int lane) {
    const int k = (t - wave) / nw;
    if ((k >> 6) != win) {
      load(a, k >> 6, lane);
      // wait here, in the rare refill, so that `ids` is never a pending load
      // where this path joins the common one (which must not wait at all)
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    return __builtin_amdgcn_readlane(ids, k & 63);
  }
};

template <int VD, int NT = kThreads, bool MT = false>
__device__ __forceinline__ bool split_range(const SplitArgs& a, const Work& w, int& p0, int& p1) {
  const int S = a.num_splits;
  int chunk;
  if (a.target_ctas > 0) {
    chunk = w.n_row > 0 ? (((w.npos + w.n_row - 1) / w.n_row + 15) & ~15) : 0;
    p0 = w.split * chunk;
  } else {
    chunk = a.static_chunk;
    p0 = static_p0(a, w.split);
  }
  p1 = min(w.npos, p0 + chunk);
  float2* const ml = reinterpret_cast<float2*>(a.ws_ml);
  if (a.target_ctas > 0 && w.split == w.n_row - 1) {
    // the row's last split also publishes the splits n_row .. S-1, which have
    // no CTA in this mode
    for (int e = threadIdx.x; e < w.nh * (S - w.n_row); e += NT)
      ml[head_slot<MT>(a, w, e % w.nh).pair * S + w.n_row + e / w.nh] = make_float2(kNegInf, 0.0f);
  }
  if (p0 >= w.npos || (a.target_ctas > 0 && w.split >= w.n_row)) {
    if (a.direct) {
      // an empty row: O = 0, lse = -inf
      for (int e = threadIdx.x; e < w.nh * (VD / 4); e += NT)
        store_final<VD>(a, head_slot<MT>(a, w, e / (VD / 4)).pair, 4 * (e % (VD / 4)),
                        make_float4(0.f, 0.f, 0.f, 0.f), 0.0f);
      if (a.lse_out && threadIdx.x < w.nh) a.lse_out[head_slot<MT>(a, w, threadIdx.x).pair] = kNegInf;
    } else if (threadIdx.x < w.nh) {
      ml[head_slot<MT>(a, w, threadIdx.x).pair * S + w.split] = make_float2(kNegInf, 0.0f);
    }
    return false;
  }
  return true;
}

// Q' = fp16(Q * k_scale) in MFMA B-operand order (shared by the CTA's waves):
// entry (ks, lane) holds channels d0(ks, lane>>4) .. +7 of head lane&15 of
// the CTA's head block.  q_issue loads the raw query, q_stage scales,
// rounds and stores it.
template <int EB>
__device__ __forceinline__ int q_channel(int ks, int lj) {
  if constexpr (EB == 2) return 32 * ks + 8 * lj;
  else return 64 * (ks >> 1) + 16 * lj + 8 * (ks & 1);
}

// With FIXED every thread issues exactly QPT query loads whatever its head
// slot (a slot past the unit's heads, or an entry past the stage, reads past
// the descriptor of the row's query block, which returns zeros without a
// memory request).  With a load count that does not depend on the path, the
// compiler's wait for the block ids before the first K tile counts these
// loads and does not wait for them (C3-shaped steps 1.6 % faster).  The
// latent kernel keeps FIXED = false: on one-byte dense rows it issues its K
// tiles as direct-to-LDS loads, which the compiler does not count, so the
// query must land before they go out (its Q' stage would otherwise wait for
// a whole round of K, measured 1.3 us slower on C5).
template <int NKS, int EB, int D, int QPT, int NT = kThreads, bool MT = false, bool FIXED = true>
__device__ __forceinline__ void q_issue(const SplitArgs& a, const Work& w, uint4 (&qraw)[QPT],
                                        float4 (&ksc)[QPT][2]) {
  if constexpr (FIXED) {
    const size_t q0 = (size_t)w.r * (MT ? a.qtok : 1) * a.heads;  // the row's first query pair
    const auto qrs = make_rsrc(a.query + q0 * D, (uint32_t)((MT ? a.qtok : 1) * a.heads * D * 2));
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + i * NT;
      ksc[i][0] = ksc[i][1] = make_float4(1.f, 1.f, 1.f, 1.f);
      const int ks = e >> 6, el = e & 63, eli = el & 15, elj = el >> 4;
      const int d0 = q_channel<EB>(ks, elj);
      const bool live = e < NKS * 64 && eli < w.nh;
      const uint32_t off =
          live ? (uint32_t)((head_slot<MT>(a, w, eli).pair - q0) * D + d0) * 2u : kPastDescriptor;
      buffer_bytes<16>(qrs, off, 0, reinterpret_cast<uint32_t*>(&qraw[i]));
      if (e < NKS * 64 && a.k_quant == PKV_QUANT_PER_CHANNEL) {
        const float4* kp = reinterpret_cast<const float4*>(a.k_scale + (size_t)w.g * D + d0);
        ksc[i][0] = kp[0];
        ksc[i][1] = kp[1];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + i * NT;
      qraw[i] = uint4{0u, 0u, 0u, 0u};
      ksc[i][0] = ksc[i][1] = make_float4(1.f, 1.f, 1.f, 1.f);
      if (e < NKS * 64) {
        const int ks = e >> 6, el = e & 63, eli = el & 15, elj = el >> 4;
        const int d0 = q_channel<EB>(ks, elj);
        if (eli < w.nh)
          qraw[i] = *reinterpret_cast<const uint4*>(a.query + head_slot<MT>(a, w, eli).pair * D + d0);
        if (a.k_quant == PKV_QUANT_PER_CHANNEL) {
          const float4* kp = reinterpret_cast<const float4*>(a.k_scale + (size_t)w.g * D + d0);
          ksc[i][0] = kp[0];
          ksc[i][1] = kp[1];
        }
      }
    }
  }
}

// ks_tensor: the per-tensor key scale (1 when not per tensor).
template <int NKS, int EB, int D, int QPT, int NT = kThreads>
__device__ __forceinline__ void q_stage(const uint4 (&qraw)[QPT], const float4 (&ksc)[QPT][2],
                                        float ks_tensor, uint4* s_q, float* s_err) {
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int e = threadIdx.x + i * NT;
    if (e < NKS * 64) {
      const half8 q = __builtin_bit_cast(half8, qraw[i]);
      const float kc[8] = {ksc[i][0].x, ksc[i][0].y, ksc[i][0].z, ksc[i][0].w,
                           ksc[i][1].x, ksc[i][1].y, ksc[i][1].z, ksc[i][1].w};
      half8 o;
      float err = 0.0f;  // folding error of the entry's eight channels
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float v = (float)q[x] * (kc[x] * ks_tensor);
        o[x] = (half_t)v;
        err += fabsf((float)o[x] - v);
      }
      s_q[e] = __builtin_bit_cast(uint4, o);
      s_err[e] = err;
    }
  }
}

// Scales read in the prologue, so the epilogue issues no dependent load:
// per-tensor values in SGPRs, per-channel value scales of the KV head
// loaded into registers (vs) and copied to LDS with the query (stage_scales).
struct Scales {
  float k_tensor;  // per-tensor key scale, else 1
  float v_tensor;  // per-tensor value scale, else 1
  float4 vs;       // this thread's float4 of the per-channel value scales
};

template <int VD, int NT = kThreads>
__device__ __forceinline__ Scales load_scales(const SplitArgs& a, int g) {
  static_assert(VD / 4 <= NT, "one float4 of value scales per thread");
  Scales sc;
  sc.k_tensor = a.k_quant == PKV_QUANT_PER_TENSOR ? uniform_load(a.k_scale, 0) : 1.0f;
  sc.v_tensor = a.v_quant == PKV_QUANT_PER_TENSOR ? uniform_load(a.v_scale, 0) : 1.0f;
  sc.vs = make_float4(1.f, 1.f, 1.f, 1.f);
  if (a.v_quant == PKV_QUANT_PER_CHANNEL && threadIdx.x < VD / 4)
    sc.vs = *reinterpret_cast<const float4*>(a.v_scale + (size_t)g * a.v_scale_stride + 4 * threadIdx.x);
  return sc;
}

template <int VD, int NT = kThreads>
__device__ __forceinline__ void stage_scales(const SplitArgs& a, const Scales& sc, float* s_vs) {
  if (a.v_quant == PKV_QUANT_PER_CHANNEL && threadIdx.x < VD / 4)
    reinterpret_cast<float4*>(s_vs)[threadIdx.x] = sc.vs;
}

// Value scale of channel c (applied once, after accumulation); s_vs holds
// the per-channel scales of the CTA's KV head.
__device__ __forceinline__ float v_scale_of(const SplitArgs& a, const Scales& sc, const float* s_vs,
                                            int c) {
  return a.v_quant == PKV_QUANT_PER_CHANNEL ? s_vs[c] : sc.v_tensor;
}

// ---- FP32 path of one work item (robust numerics) ----------------------------
//
// Recomputes the partial of the CTA's work item from the definition, one
// query head at a time: every wave takes the positions p0 + wave + W j, the
// score is the FP32 dot product of the unfolded Q k_scale with the exactly
// decoded key codes (reduced across the wave), the running maximum is exact
// (natural-log units), and the FP32 accumulator is multiplied by the value
// scale after the W wave states are merged in a fixed order.  `scratch`
// holds W * (VD + 2) floats of LDS; every thread of the CTA calls this.
template <int CT, int D, int VD, bool LATENT, bool GATHER, int W, bool EXT, bool MT = false>
__device__ __forceinline__ void exact_partial(const SplitArgs& a, const Work& wk, int p0, int p1,
                                           const Scales& sc, const float* s_vs, float* scratch) {
  constexpr int NT = 64 * W;
  constexpr int EB = (CT == PKV_F16) ? 2 : 1;
  constexpr int KROW = D * EB;
  constexpr int VROW = LATENT ? KROW : VD * EB;
  constexpr int KD = (D + 63) / 64;
  constexpr int KV = (VD + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.num_splits;
  const int KVH = a.kv_heads;
  const int g = wk.g;
  const int32_t* bt_row = a.block_table + (size_t)wk.r * a.max_blocks_per_row;
  const uint8_t* vbase = LATENT ? a.key_cache : a.value_cache;
  for (int hh = 0; hh < wk.nh; ++hh) {
    const HeadSlot hs = head_slot<MT>(a, wk, hh);
    const int h = hs.h;
    // (several tokens per row: token j sees len - T + 1 + j positions, and
    // with a sliding window the last `window` of them)
    const int tlen = MT ? wk.len - (a.qtok - 1 - hs.tok) : wk.len;
    const int tlo = (MT && a.window > 0 && tlen > a.window) ? tlen - a.window : wk.lo;
    float qf[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const int d = lane + 64 * k;
      qf[k] = 0.0f;
      if (d < D) {
        const float ks = a.k_quant == PKV_QUANT_PER_CHANNEL ? a.k_scale[(size_t)g * D + d] : sc.k_tensor;
        qf[k] = (float)reinterpret_cast<const half_t*>(a.query)[hs.pair * D + d] * ks;
      }
    }
    float m = kNegInf, l = 0.0f;
    float acc[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) acc[k] = 0.0f;
    for (int pos = p0 + wave; pos < p1; pos += W) {
      int t = wk.base + pos;
      if constexpr (GATHER) t = a.candidates[(size_t)wk.r * a.max_candidates + pos];
      if (t < tlo || t >= tlen) continue;
      const int blk = bt_row[t >> a.log2_block];
      if (blk < 0 || blk >= a.num_pool_blocks) continue;
      const size_t slot = ((size_t)blk << a.log2_block) + (t & (a.block_size - 1));
      const uint8_t* krow = a.key_cache + (slot * KVH + g) * KROW;
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        const int d = lane + 64 * k;
        if (d < D) part += qf[k] * code_at<CT>(krow, d);
      }
      const float sv = soft_cap<EXT>(a, wave_sum(part) * a.score_scale);
      if (sv > m) {
        const float alpha = (m == kNegInf) ? 0.0f : expf(m - sv);
        l *= alpha;
#pragma unroll
        for (int k = 0; k < KV; ++k) acc[k] *= alpha;
        m = sv;
      }
      const float pp = expf(sv - m);
      l += pp;
      const uint8_t* vrow = vbase + (slot * KVH + g) * VROW;
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const int c = lane + 64 * k;
        if (c < VD) acc[k] += pp * code_at<CT>(vrow, c);
      }
    }
    float* sw = scratch + wave * (VD + 2);
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int c = lane + 64 * k;
      if (c < VD) sw[c] = acc[k];
    }
    if (lane == 0) {
      sw[VD] = m;
      sw[VD + 1] = l;
    }
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, scratch[w * (VD + 2) + VD]);
    float f[W];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = scratch[w * (VD + 2) + VD];
      f[w] = (mw == kNegInf) ? 0.0f : expf(mw - M);
      L += f[w] * scratch[w * (VD + 2) + VD + 1];
    }
    const size_t pidx = hs.pair * S + wk.split;
    if (a.direct) {
      const Final fin = final_of(a, h, M, L);
      const size_t pair = hs.pair;
      for (int c4 = threadIdx.x; c4 < VD / 4; c4 += NT) {
        float part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * c4 + j;
          float o = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) o += f[w] * scratch[w * (VD + 2) + c];
          part[j] = o * v_scale_of(a, sc, s_vs, c);
        }
        store_final<VD>(a, pair, 4 * c4, make_float4(part[0], part[1], part[2], part[3]), fin.f);
      }
      if (a.lse_out && threadIdx.x == 0) a.lse_out[pair] = fin.lse;
    } else {
      for (int c = threadIdx.x; c < VD; c += NT) {
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) o += f[w] * scratch[w * (VD + 2) + c];
        a.ws_acc[pidx * VD + c] = o * v_scale_of(a, sc, s_vs, c);
      }
      if (threadIdx.x == 0) reinterpret_cast<float2*>(a.ws_ml)[pidx] = make_float2(M, L);
    }
    __syncthreads();
  }
}

// Folding bound of the CTA's heads (called by one wave after Q' is staged):
// true when some head's eps_h exceeds the budget.  s_err holds, per Q'
// entry, the summed |fp16(Q ks) - Q ks| of its eight channels.
template <int CT, int NKS>
__device__ __forceinline__ bool fold_over_budget(const SplitArgs& a, const float* s_err, int nh,
                                                 int lane) {
  float e = 0.0f;
  if (lane < 16 && lane < nh) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int lj = 0; lj < 4; ++lj) e += s_err[ks * 64 + lj * 16 + lane];
  }
  return __any(e * code_bound<CT>() * a.score_scale > kFoldBudget);
}

// max |value| of the KV head's quantised values (0 when V is not quantised)
template <int CT, int VD>
__device__ __forceinline__ float value_bound(const SplitArgs& a, const Scales& sc, const float* s_vs,
                                             int lane) {
  if (a.v_quant == PKV_QUANT_NONE) return 0.0f;
  float vm = fabsf(sc.v_tensor);
  if (a.v_quant == PKV_QUANT_PER_CHANNEL) {
    vm = 0.0f;
    for (int c = lane; c < VD; c += 64) vm = fmaxf(vm, fabsf(s_vs[c]));
    vm = wave_max(vm);
  }
  return vm * code_bound<CT>();
}

template <int CT, int D, int VD, bool LATENT, bool GATHER, bool EXT, bool MT>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(SplitCfg<CT, D, VD, LATENT, GATHER>::MIN_WAVES)))
split_kernel(const SplitArgs a) {
  using C = SplitCfg<CT, D, VD, LATENT, GATHER>;
  constexpr int W = kWaves;
  constexpr int NST = C::NST;
  const int lane = threadIdx.x & 63;
  // wave index as a wave-uniform (scalar) value, so everything derived from
  // it -- tile positions, block ids, buffer descriptors -- lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;      // MFMA row/column index of this lane
  const int lj = lane >> 4;      // MFMA k-group of this lane

  const int S = a.num_splits;
  const int KVH = a.kv_heads;
  // ---- prologue: every independent read is issued before the first wait
  // (static mode: row length, first block ids, scales and query together)
  const bool balanced = a.target_ctas > 0;
  Work wk;
  int raw_npos = 0, raw_len = 0;
  if (balanced) {
    if (!locate_balanced<GATHER, EXT>(a, lane, wk)) return;  // padding CTA
  } else {
    static_item(a, wk);
    raw_npos = GATHER ? uniform_load(a.num_candidates, wk.r) : uniform_load(a.seq_lens, wk.r);
  }
  if constexpr (GATHER) raw_len = uniform_load(a.seq_lens, wk.r);
  unit_heads<MT>(a, wk);
  const int r = wk.r, g = wk.g, nh = wk.nh;

  __shared__ uint4 s_q[C::NKS * 64];
  __shared__ float s_err[C::NKS * 64];  // folding error per Q' entry
  __shared__ int s_flag[W + 1];         // per wave: a deep-tail probability; [W]: folding
  __shared__ float s_vs[VD];
  constexpr int QPT = (C::NKS * 64 + kThreads - 1) / kThreads;  // entries per thread
  uint4 qraw[QPT];
  float4 ksc[QPT][2];
  const int32_t* bt_row = a.block_table + (size_t)r * a.max_blocks_per_row;
  // block ids of this wave's first 64 tiles (static mode: before the length;
  // read again below when a sliding window moves the row's first token)
  WaveBlocks wb{bt_row, wk.base + split_p0(a, wk), wave, W, 0, 0};
  if constexpr (!GATHER) wb.load(a, 0, lane);
  q_issue<C::NKS, C::EB, D, QPT, kThreads, MT>(a, wk, qraw, ksc);
  const Scales sc = load_scales<VD>(a, g);
  finish_item<GATHER, EXT>(a, wk, balanced, raw_npos, raw_len);
  const int len = wk.len;
  if constexpr (!GATHER && EXT)
    if (!balanced && wk.base > 0) {
      wb.p0 = wk.base + split_p0(a, wk);
      wb.load(a, 0, lane);
    }
  // positions of the row before its window start (first tile only)
  const int skip = wk.lo - wk.base;
  const int base = wk.base;
  const int lo = wk.lo;

  int p0, p1;
  if (!split_range<VD, kThreads, MT>(a, wk, p0, p1)) return;
  const int split = wk.split;
  const int ntiles = (p1 - p0 + 15) >> 4;
  // several tokens per row: positions of this lane's head slot (its token
  // sees T - 1 - j fewer than the row's last)
  int lim = p1;
  if constexpr (MT) lim = li < nh ? wk.npos - (a.qtok - 1 - head_slot<MT>(a, wk, li).tok) : p1;

  // Per-lane byte offsets inside a 16-token tile of one block (dense rows):
  // K: row of token li, 16-byte chunk lj (+64 s);  V: rows of tokens 4 lj + q
  // (q times the token stride), segment li.
  const uint32_t tok_k = (uint32_t)KVH * C::KROW;                  // bytes per token slot (K)
  const uint32_t tok_v = (uint32_t)KVH * (LATENT ? C::KROW : C::VROW);
  const uint32_t koff = (uint32_t)li * tok_k + (uint32_t)g * C::KROW + 16u * lj;
  const uint32_t voff = (uint32_t)(4 * lj) * tok_v + (uint32_t)g * (LATENT ? C::KROW : C::VROW) +
                        (uint32_t)li * C::VSEG;

  // Issue the loads of tile t into T.  Tiles at or past ntiles issue loads
  // that read nothing (dense rows: an empty buffer descriptor) so every
  // iteration issues the same instruction stream.
  auto issue = [&](Tile<C>& T, int t) __attribute__((always_inline)) {
    const int tp = p0 + 16 * t;  // first position of the tile
    uint32_t vm = 0;
    if constexpr (!GATHER) {
      int blk = 0;
      bool bv = false;
      if (t < ntiles) {
        // the address is wave-uniform; keep the block id in an SGPR
        blk = wb.of(a, t, lane);
        bv = blk >= 0 && blk < a.num_pool_blocks;
      }
      const int64_t s0 =
          bv ? ((int64_t)blk << a.log2_block) + ((base + tp) & (a.block_size - 1)) : 0;
      // the descriptors cover the tile's valid rows only: rows past the end
      // (and a whole tile with an invalid block) read as zeros, so the V
      // operands need no mask; rows before a sliding window's start (first
      // tile only) get an offset past the descriptor and read as zeros too
      const uint32_t nv = bv ? (uint32_t)min(16, p1 - tp) : 0u;
      const auto krs = make_rsrc(a.key_cache + s0 * tok_k, nv * tok_k);
#pragma unroll
      for (int s = 0; s < C::NKL; ++s) buffer_bytes<16>(krs, koff + 64 * s, 0, &T.k[4 * s]);
      const uint8_t* vbase = LATENT ? a.key_cache : a.value_cache;
      const auto vrs = make_rsrc(vbase + s0 * tok_v, nv * tok_v);
      if (EXT && tp < skip) {
        // the row's first tile under a sliding window: its rows before the
        // window start are masked and their V reads go past the descriptor
        const int sk = skip - tp;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * lj + q;
          const uint32_t past = row < sk ? kPastDescriptor : 0u;
          buffer_bytes<C::VSEG>(vrs, voff + (uint32_t)q * tok_v + past, 0, T.v[q]);
          vm |= (row < (int)nv && row >= sk) ? (1u << q) : 0u;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          buffer_bytes<C::VSEG>(vrs, voff + (uint32_t)q * tok_v, 0, T.v[q]);
          vm |= (4 * lj + q < (int)nv) ? (1u << q) : 0u;
        }
      }
    } else {
      // gathered rows: per-token slots; invalid entries (and tiles past the
      // end) read token slot 0 of the pool and are masked
      const int pos = tp + li;
      int c = (t < ntiles && pos < p1) ? a.candidates[(size_t)r * a.max_candidates + pos] : -1;
      bool v = c >= lo && c < len;
      int blk = v ? bt_row[c >> a.log2_block] : 0;
      v = v && blk >= 0 && blk < a.num_pool_blocks;
      const int64_t s = v ? ((int64_t)blk << a.log2_block) + (c & (a.block_size - 1)) : 0;
      const uint8_t* krow = a.key_cache + ((size_t)s * KVH + g) * C::KROW;
#pragma unroll
      for (int i = 0; i < C::NKL; ++i) load_bytes<16>(krow + 64 * i + 16 * lj, &T.k[4 * i]);
      const int vi = v ? 1 : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int src = 4 * lj + q;
        const int lo = __shfl((int)(s & 0xffffffff), src);
        const int hi = __shfl((int)(s >> 32), src);
        const int64_t sq = ((int64_t)hi << 32) | (uint32_t)lo;
        const uint8_t* vrow;
        if constexpr (LATENT) vrow = a.key_cache + ((size_t)sq * KVH + g) * C::KROW;
        else vrow = a.value_cache + ((size_t)sq * KVH + g) * C::VROW;
        load_bytes<C::VSEG>(vrow + li * C::VSEG, T.v[q]);
        vm |= __shfl(vi, src) ? (1u << q) : 0u;
      }
    }
    T.vmask = vm;
  };

  // ---- per-wave state -----------------------------------------------------
  f32x4 acc[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // running reference maximum of head li (natural log units)
  float l_part = 0.0f;     // this lane's share of the running sum
  float smin = __builtin_inff();  // smallest valid score of this lane (tail-depth check)

  // Consume tile T: scores, online softmax, PV (lo: with the residual
  // probability tile).
  auto consume = [&](const Tile<C>& T, int tt, auto lo) __attribute__((always_inline)) {
    constexpr bool LO = decltype(lo)::value;
    // S^T = K Q'^T : lane holds scores of tokens 4 lj + q for head li
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) {
      if constexpr (C::EB == 2) {
        const half8 kop = __builtin_bit_cast(
            half8, uint4{T.k[4 * s], T.k[4 * s + 1], T.k[4 * s + 2], T.k[4 * s + 3]});
        const half8 qop = __builtin_bit_cast(half8, s_q[s * 64 + lane]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop, sacc, 0, 0, 0);
      } else {
        const half4 c0 = codes4_to_half4<CT>(T.k[4 * s + 0]);
        const half4 c1 = codes4_to_half4<CT>(T.k[4 * s + 1]);
        const half4 c2 = codes4_to_half4<CT>(T.k[4 * s + 2]);
        const half4 c3 = codes4_to_half4<CT>(T.k[4 * s + 3]);
        const half8 k0 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const half8 k1 = {c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
        const half8 q0 = __builtin_bit_cast(half8, s_q[(2 * s) * 64 + lane]);
        const half8 q1 = __builtin_bit_cast(half8, s_q[(2 * s + 1) * 64 + lane]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q0, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q1, sacc, 0, 0, 0);
      }
    }
    float sc[4];
    scaled_scores<EXT>(a, sacc, sc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bool valid = (T.vmask >> q) & 1u;
      if constexpr (MT) {
        const int pos = p0 + 16 * tt + 4 * lj + q;
        valid = valid && pos < lim;
        // the slot's own window start (the row's range starts at the first
        // token's)
        if constexpr (EXT) valid = valid && (a.window == 0 || pos >= lim - a.window);
      } else {
        (void)tt;
      }
      sc[q] = valid ? sc[q] : kNegInf;
      smin = fminf(smin, valid ? sc[q] : __builtin_inff());
    }
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
    half4 pop, pol;  // FP16(16 p) and its residual
    split_prob<LO>(p, pop, pol);

    // V^T operands: for col tile ct, lane holds channel li*CPL+ct of tokens
    // 4 lj .. 4 lj + 3 (rows q = 0..3 of its segments), transposed in registers
    uint32_t vz[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vz[q] = (GATHER && !((T.vmask >> q) & 1u)) ? 0u : 0xffffffffu;
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
        if constexpr (LO) {
          acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pol, acc[2 * w], 0, 0, 0);
          acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vb, pol, acc[2 * w + 1], 0, 0, 0);
        }
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
        const half4 h0 = codes4_to_half4<CT>(o0), h1 = codes4_to_half4<CT>(o1);
        const half4 h2 = codes4_to_half4<CT>(o2), h3 = codes4_to_half4<CT>(o3);
        acc[4 * w + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(h0, pop, acc[4 * w + 0], 0, 0, 0);
        acc[4 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(h1, pop, acc[4 * w + 1], 0, 0, 0);
        acc[4 * w + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(h2, pop, acc[4 * w + 2], 0, 0, 0);
        acc[4 * w + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(h3, pop, acc[4 * w + 3], 0, 0, 0);
        if constexpr (LO) {
          acc[4 * w + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(h0, pol, acc[4 * w + 0], 0, 0, 0);
          acc[4 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(h1, pol, acc[4 * w + 1], 0, 0, 0);
          acc[4 * w + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(h2, pol, acc[4 * w + 2], 0, 0, 0);
          acc[4 * w + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(h3, pol, acc[4 * w + 3], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop: wave `wave` takes tiles wave, wave + W, ...; NST - 1
  // tiles in flight while one is consumed -----------------------------------
  Tile<C> buf[NST];
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) issue(buf[i], wave + i * W);

  // Q' into LDS (its loads were issued before the tile loads above)
  q_stage<C::NKS, C::EB, D>(qraw, ksc, sc.k_tensor, s_q, s_err);
  stage_scales<VD>(a, sc, s_vs);
  __syncthreads();
  // folding bound of the CTA's heads (read after the final barrier)
  if (wave == 0) {
    const bool fold = fold_over_budget<CT, C::NKS>(a, s_err, nh, lane);
    if (lane == 0) s_flag[W] = fold ? 1 : 0;
  }

  auto tile_loop = [&](auto lo) __attribute__((always_inline)) {
    for (int t = wave; t < ntiles; t += NST * W) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int tt = t + st * W;
        if (tt >= ntiles) break;
        issue(buf[(st + NST - 1) % NST], tt + (NST - 1) * W);
        // keep the loads ahead of the wait for this tile's data
        __builtin_amdgcn_sched_barrier(0);
        consume(buf[st], tt, lo);
      }
    }
  };
  tile_loop(std::integral_constant<bool, kResidualTile>{});
  // a valid probability that fell below the FP16 tile's normal range: some
  // score more than ln 2^18 below the lane's final reference maximum (the
  // reference never decreases, so this is conservative)
  const bool deep = smin != __builtin_inff() && smin - m_ref < kTailLog;

  // ---- merge the W wave states (fixed order) and publish the partial -----
  // l: sum the four lane groups of head li
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);

  // Flat merge: every wave writes its rescaled accumulator to LDS, and after
  // one barrier every thread sums the four wave slices (fixed order) for a
  // strided set of float4 channel groups of one head and writes them -- the
  // partial store is spread over the whole CTA and fully coalesced.
  __shared__ float sm_m[W][16];
  __shared__ float sm_l[W][16];
  constexpr int HS = VD + 4;  // padded head stride (floats): conflict-free float4 writes
  __shared__ __attribute__((aligned(16))) float sm_acc[W * 16 * HS];

  if (lane < 16) {
    sm_m[wave][lane] = m_ref;
    sm_l[wave][lane] = l_part;
  }
  {
    const bool dw = __any(deep);
    if (lane == 0) s_flag[wave] = dw ? 1 : 0;
  }
  __syncthreads();
  {
    // robust numerics: recompute on the FP32 path when the folding bound or
    // the tail-depth check fails (a CTA-uniform decision)
    bool deep_any = false;
#pragma unroll
    for (int w = 0; w < W; ++w) deep_any |= s_flag[w] != 0;
    const bool armed = deep_any && value_bound<CT, VD>(a, sc, s_vs, lane) * (float)(p1 - p0) >= kTailArm;
    if (s_flag[W] != 0 || (deep_any && armed)) {
      exact_partial<CT, D, VD, LATENT, GATHER, W, EXT, MT>(a, wk, p0, p1, sc, s_vs, sm_acc);
      return;
    }
  }
  {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][li]);
    const float f = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - M) * kLog2e);
    // lane holds channels (4 lj + q) * CPL + ct of head li
    float* dst = sm_acc + (size_t)(wave * 16 + li) * HS;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int ct = 0; ct < C::NCT; ct += 4)
        *reinterpret_cast<float4*>(dst + (4 * lj + q) * C::CPL + ct) =
            make_float4(acc[ct][q] * f, acc[ct + 1][q] * f, acc[ct + 2][q] * f, acc[ct + 3][q] * f);
  }
  __syncthreads();
  {
    const int hh = threadIdx.x >> 4;  // head of the CTA's block
    const int cc = threadIdx.x & 15;  // float4 groups cc, cc + 16, ...
    if (hh < nh) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][hh]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sm_m[w][hh];
        L += ((mw == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((mw - M) * kLog2e)) * sm_l[w][hh];
      }
      const HeadSlot hs = head_slot<MT>(a, wk, hh);
      const size_t pidx = hs.pair * S + split;
      const size_t pair = hs.pair;
      Final fin{0.0f, kNegInf};
      if (a.direct) {
        fin = final_of(a, hs.h, M, L);
        if (a.lse_out && cc == 0) a.lse_out[pair] = fin.lse;
      } else if (cc == 0) {
        reinterpret_cast<float2*>(a.ws_ml)[pidx] = make_float2(M, L);
      }
      float* dst = a.ws_acc + pidx * VD;
#pragma unroll
      for (int j = 0; j < VD / 64; ++j) {
        const int c = 4 * (cc + 16 * j);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float4 v = *reinterpret_cast<const float4*>(sm_acc + (size_t)(w * 16 + hh) * HS + c);
          o.x += v.x;
          o.y += v.y;
          o.z += v.z;
          o.w += v.w;
        }
        // value scale applied once, after accumulation
        o.x *= a.v_mult * v_scale_of(a, sc, s_vs, c);
        o.y *= a.v_mult * v_scale_of(a, sc, s_vs, c + 1);
        o.z *= a.v_mult * v_scale_of(a, sc, s_vs, c + 2);
        o.w *= a.v_mult * v_scale_of(a, sc, s_vs, c + 3);
        if (a.direct)
          store_final<VD>(a, pair, c, o, fin.f);
        else
          *reinterpret_cast<float4*>(dst + c) = o;
      }
    }
  }
}

constexpr int kKvpWavesPerSimd = 2;

// ---- four KV heads per CTA (dense rows, separate K / V caches) -------------
//
// The cache keeps the rows of all KV heads of a token side by side
// ([block, token, kv_head, dim]).  A CTA per KV head reads only its slice of
// every token record, at its own pace; on MI355X a streaming probe reads
// such per-head slices at 5.4-5.6 TB/s, but 6.3 TB/s when the four waves of
// one CTA read four neighbouring slices of the same records together.  So
// when a problem has a multiple of four KV heads, one CTA takes KV heads
// 4u .. 4u + 3 of a row and split: wave w takes KV head 4u + w and every
// tile of the split's range, with split_kernel's per-tile code (gather,
// exact conversion, MFMA scores, online softmax, PV) for VB 16-slot head
// blocks of its KV head (VB = 2 for 17-32 (token, head) slots: both MFMA
// column tiles share each K / V tile the wave loads and converts, so every
// KV byte is read once for all slots).  Each wave holds the complete state
// of its slots, so the waves need no merge: every wave writes its own
// partials straight from registers.
//
// Several CTAs share a CU, and the sequencer issues the oldest wave first,
// so with equal priorities the CTAs dispatched last to a CU starved: on the
// C3 continuous-batching workload the third CTA of a CU waited 25-30 us
// for its first data, and the kernel ended with a long tail of lone CTAs
// reading with little in flight.  So every wave runs its prologue at the
// highest priority and then lowers its priority as its remaining work
// shrinks (3, 2, 1, 0 for the quarters of its tiles): the CTAs of a CU
// progress together and finish together.  Two tiles stay in flight per wave
// for head-128 FP16 tiles, at two waves per SIMD (measured better than one
// tile at three waves per SIMD once the priorities are set), one for smaller
// tiles (see NST).

template <int CT, int D, int VD, bool EXT, int KPC, bool MT, int VB>
__global__ void __launch_bounds__(64 * KPC)
__attribute__((amdgpu_waves_per_eu(kKvpWavesPerSimd)))
split_kvp_kernel(const SplitArgs a) {
  __builtin_amdgcn_s_setprio(3);
  using C = SplitCfg<CT, D, VD, false, false>;
  static_assert(VB == 1 || VB == 2, "one or two 16-slot head blocks per wave");
  constexpr int W = KPC;       // KV heads per CTA, one per wave
  constexpr int NT = 64 * W;   // threads per CTA
  // tiles held per wave: one consumed, two in flight -- or one for tiles of
  // at most 16 registers (one-byte codes up to head 128, FP16 head 64), where
  // the registers saved raise the CTAs per CU (measured on MI355X: the
  // PagedAttention 16384-token x 32-row shapes 5 % faster, C3 with head 64
  // 2 %, the rest unchanged; one tile in flight for head-128 FP16 was slower)
  constexpr int NST = C::TILE_REGS <= 16 ? 2 : 3;
  static_assert(C::CPL % 4 == 0, "float4 groups of channels per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int lj = lane >> 4;
  const int S = a.num_splits;
  const int KVH = a.kv_heads;
  const int group = a.group;
  const int vgroup = MT ? a.qtok * group : group;  // head slots per KV head

  // ---- prologue (as split_kernel, for four KV heads)
  const bool balanced = a.target_ctas > 0;
  Work wk;
  int raw_npos = 0;
  if (balanced) {
    if (!locate_balanced<false, EXT>(a, lane, wk)) return;  // padding CTA
  } else {
    static_item(a, wk);
    raw_npos = uniform_load(a.seq_lens, wk.r);
  }
  // the unit: KV heads 4u .. 4u + 3 and their query heads (contiguous)
  wk.g = W * wk.u;
  wk.hb = 0;
  wk.h0 = wk.g * group;
  wk.nh = W * vgroup;
  const int r = wk.r;
  const int g = wk.g + wave;     // this wave's KV head

  // Q' of head block vb of KV head 4u + w at [w * VB + vb]
  __shared__ uint4 s_q[W * VB][C::NKS * 64];
  __shared__ float s_err[W * VB][C::NKS * 64];
  __shared__ int s_flag[2 * W];  // [w]: deep tail, [W + w]: folding, of wave w
  __shared__ float s_vs[W][VD];
  constexpr int QPT = (C::NKS * 64 + NT - 1) / NT;
  uint4 qraw[W * VB][QPT];
  float4 ksc[W * VB][QPT][2];
  Scales sc[W];
  const int32_t* bt_row = a.block_table + (size_t)r * a.max_blocks_per_row;
  // every wave walks every tile: the block ids of the split's first 64 tiles
  WaveBlocks wb{bt_row, wk.base + split_p0(a, wk), 0, 1, 0, 0};
  wb.load(a, 0, lane);
  // head block vb (slots 16 vb .. 16 vb + 15) of KV head 4u + u4
  auto unit_of = [&](int u4, int vb) __attribute__((always_inline)) {
    Work w = wk;
    w.g = wk.g + u4;
    w.hb = vb;
    w.h0 = w.g * group + (MT ? 0 : 16 * vb);
    w.nh = min(16, vgroup - 16 * vb);
    return w;
  };
#pragma unroll
  for (int u4 = 0; u4 < W; ++u4) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
      q_issue<C::NKS, C::EB, D, QPT, NT, MT>(a, unit_of(u4, vb), qraw[u4 * VB + vb], ksc[u4 * VB + vb]);
    sc[u4] = load_scales<VD, NT>(a, wk.g + u4);
  }
  finish_item<false, EXT>(a, wk, balanced, raw_npos, 0);
  const int len = wk.len;
  if constexpr (EXT)
    if (!balanced && wk.base > 0) {
      wb.p0 = wk.base + split_p0(a, wk);
      wb.load(a, 0, lane);
    }
  const int skip = wk.lo - wk.base;
  const int base = wk.base;
  (void)len;

  int p0, p1;
  if (!split_range<VD, NT, MT>(a, wk, p0, p1)) return;
  const int split = wk.split;
  const int ntiles = (p1 - p0 + 15) >> 4;
  // several tokens per row: positions of this lane's head slot
  int lim[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    lim[vb] = p1;
    if constexpr (MT)
      lim[vb] = li < min(16, vgroup - 16 * vb)
                    ? wk.npos - (a.qtok - 1 - head_slot<MT>(a, unit_of(wave, vb), li).tok)
                    : p1;
  }

  const uint32_t tok_k = (uint32_t)KVH * C::KROW;
  const uint32_t tok_v = (uint32_t)KVH * C::VROW;
  const uint32_t koff = (uint32_t)li * tok_k + (uint32_t)g * C::KROW + 16u * lj;
  const uint32_t voff = (uint32_t)(4 * lj) * tok_v + (uint32_t)g * C::VROW + (uint32_t)li * C::VSEG;

  // loads of tile t (split_kernel's dense branch)
  auto issue = [&](Tile<C>& T, int t) __attribute__((always_inline)) {
    const int tp = p0 + 16 * t;
    uint32_t vm = 0;
    int blk = 0;
    bool bv = false;
    if (t < ntiles) {
      blk = wb.of(a, t, lane);
      bv = blk >= 0 && blk < a.num_pool_blocks;
    }
    const int64_t s0 = bv ? ((int64_t)blk << a.log2_block) + ((base + tp) & (a.block_size - 1)) : 0;
    const uint32_t nv = bv ? (uint32_t)min(16, p1 - tp) : 0u;
    const auto krs = make_rsrc(a.key_cache + s0 * tok_k, nv * tok_k);
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) buffer_bytes<16>(krs, koff + 64 * s, 0, &T.k[4 * s]);
    const auto vrs = make_rsrc(a.value_cache + s0 * tok_v, nv * tok_v);
    if (EXT && tp < skip) {
      const int sk = skip - tp;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 4 * lj + q;
        const uint32_t past = row < sk ? kPastDescriptor : 0u;
        buffer_bytes<C::VSEG>(vrs, voff + (uint32_t)q * tok_v + past, 0, T.v[q]);
        vm |= (row < (int)nv && row >= sk) ? (1u << q) : 0u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        buffer_bytes<C::VSEG>(vrs, voff + (uint32_t)q * tok_v, 0, T.v[q]);
        vm |= (4 * lj + q < (int)nv) ? (1u << q) : 0u;
      }
    }
    T.vmask = vm;
  };

  // per head block: accumulator, running maximum and sum of the lane's head
  // slot, smallest valid score
  f32x4 acc[VB][C::NCT];
  float m_ref[VB], l_part[VB], smin[VB];
  const uint4* sq[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) acc[vb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[vb] = kNegInf;
    l_part[vb] = 0.0f;
    smin[vb] = __builtin_inff();
    sq[vb] = s_q[wave * VB + vb];
  }

  // split_kernel's tile consumer, on this wave's query block
  auto consume = [&](const Tile<C>& T, int tt, auto lo) __attribute__((always_inline)) {
    constexpr bool LO = decltype(lo)::value;
    f32x4 sacc[VB];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) sacc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) {
      if constexpr (C::EB == 2) {
        const half8 kop = __builtin_bit_cast(
            half8, uint4{T.k[4 * s], T.k[4 * s + 1], T.k[4 * s + 2], T.k[4 * s + 3]});
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const half8 qop = __builtin_bit_cast(half8, sq[vb][s * 64 + lane]);
          sacc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop, sacc[vb], 0, 0, 0);
        }
      } else {
        const half4 c0 = codes4_to_half4<CT>(T.k[4 * s + 0]);
        const half4 c1 = codes4_to_half4<CT>(T.k[4 * s + 1]);
        const half4 c2 = codes4_to_half4<CT>(T.k[4 * s + 2]);
        const half4 c3 = codes4_to_half4<CT>(T.k[4 * s + 3]);
        const half8 k0 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const half8 k1 = {c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const half8 q0 = __builtin_bit_cast(half8, sq[vb][(2 * s) * 64 + lane]);
          const half8 q1 = __builtin_bit_cast(half8, sq[vb][(2 * s + 1) * 64 + lane]);
          sacc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q0, sacc[vb], 0, 0, 0);
          sacc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q1, sacc[vb], 0, 0, 0);
        }
      }
    }
    half4 pop[VB], pol[VB];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      float x[4];
      scaled_scores<EXT>(a, sacc[vb], x);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bool valid = (T.vmask >> q) & 1u;
        if constexpr (MT) {
          const int pos = p0 + 16 * tt + 4 * lj + q;
          valid = valid && pos < lim[vb];
          if constexpr (EXT) valid = valid && (a.window == 0 || pos >= lim[vb] - a.window);
        } else {
          (void)tt;
        }
        x[q] = valid ? x[q] : kNegInf;
        smin[vb] = fminf(smin[vb], valid ? x[q] : __builtin_inff());
      }
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__any(mt > m_ref[vb] + kRescaleSlack)) {
        const float mn = fmaxf(m_ref[vb], mt);
        const float alpha =
            (m_ref[vb] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref[vb] - mn) * kLog2e);
        l_part[vb] *= alpha;
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) acc[vb][ct] *= alpha;
        m_ref[vb] = mn;
      }
      const float mu = (m_ref[vb] == kNegInf) ? 0.0f : m_ref[vb];
      float p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = __builtin_amdgcn_exp2f((x[q] - mu) * kLog2e);
      l_part[vb] += (p[0] + p[1]) + (p[2] + p[3]);
      split_prob<LO>(p, pop[vb], pol[vb]);
    }
    if constexpr (C::EB == 2) {
#pragma unroll
      for (int w = 0; w < C::NVW; ++w) {
        const uint32_t r0 = T.v[0][w], r1 = T.v[1][w];
        const uint32_t r2 = T.v[2][w], r3 = T.v[3][w];
        const uint32_t a01 = perm(r1, r0, 0x05040100u), a23 = perm(r3, r2, 0x05040100u);
        const uint32_t b01 = perm(r1, r0, 0x07060302u), b23 = perm(r3, r2, 0x07060302u);
        const half4 va = __builtin_bit_cast(half4, uint2{a01, a23});
        const half4 vc = __builtin_bit_cast(half4, uint2{b01, b23});
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          acc[vb][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pop[vb], acc[vb][2 * w], 0, 0, 0);
          acc[vb][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vc, pop[vb], acc[vb][2 * w + 1], 0, 0, 0);
          if constexpr (LO) {
            acc[vb][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pol[vb], acc[vb][2 * w], 0, 0, 0);
            acc[vb][2 * w + 1] =
                __builtin_amdgcn_mfma_f32_16x16x16f16(vc, pol[vb], acc[vb][2 * w + 1], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < C::NVW; ++w) {
        const uint32_t r0 = T.v[0][w], r1 = T.v[1][w];
        const uint32_t r2 = T.v[2][w], r3 = T.v[3][w];
        const uint32_t t0 = perm(r1, r0, 0x05010400u), t1 = perm(r1, r0, 0x07030602u);
        const uint32_t t2 = perm(r3, r2, 0x05010400u), t3 = perm(r3, r2, 0x07030602u);
        const uint32_t o0 = perm(t2, t0, 0x05040100u), o1 = perm(t2, t0, 0x07060302u);
        const uint32_t o2 = perm(t3, t1, 0x05040100u), o3 = perm(t3, t1, 0x07060302u);
        const half4 h0 = codes4_to_half4<CT>(o0), h1 = codes4_to_half4<CT>(o1);
        const half4 h2 = codes4_to_half4<CT>(o2), h3 = codes4_to_half4<CT>(o3);
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          acc[vb][4 * w + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(h0, pop[vb], acc[vb][4 * w + 0], 0, 0, 0);
          acc[vb][4 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(h1, pop[vb], acc[vb][4 * w + 1], 0, 0, 0);
          acc[vb][4 * w + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(h2, pop[vb], acc[vb][4 * w + 2], 0, 0, 0);
          acc[vb][4 * w + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(h3, pop[vb], acc[vb][4 * w + 3], 0, 0, 0);
          if constexpr (LO) {
            acc[vb][4 * w + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(h0, pol[vb], acc[vb][4 * w + 0], 0, 0, 0);
            acc[vb][4 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(h1, pol[vb], acc[vb][4 * w + 1], 0, 0, 0);
            acc[vb][4 * w + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(h2, pol[vb], acc[vb][4 * w + 2], 0, 0, 0);
            acc[vb][4 * w + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(h3, pol[vb], acc[vb][4 * w + 3], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---- main loop: every wave walks all tiles; NST - 1 in flight
  Tile<C> buf[NST];
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) issue(buf[i], i);
#pragma unroll
  for (int u4 = 0; u4 < W; ++u4) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
      q_stage<C::NKS, C::EB, D, QPT, NT>(qraw[u4 * VB + vb], ksc[u4 * VB + vb], sc[u4].k_tensor,
                                         s_q[u4 * VB + vb], s_err[u4 * VB + vb]);
    stage_scales<VD, NT>(a, sc[u4], s_vs[u4]);
  }
  __syncthreads();
  bool fold = false;
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
    fold |= fold_over_budget<CT, C::NKS>(a, s_err[wave * VB + vb], min(16, vgroup - 16 * vb), lane);

  auto tile_loop = [&](auto lo) __attribute__((always_inline)) {
    for (int t = 0; t < ntiles; t += NST) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int tt = t + st;
        if (tt >= ntiles) break;
        issue(buf[(st + NST - 1) % NST], tt + NST - 1);
        __builtin_amdgcn_sched_barrier(0);
        {
          // priority by the share of the wave's tiles still to come
          const int pr = (4 * (ntiles - tt)) / (ntiles + 1);
          if (pr >= 3) __builtin_amdgcn_s_setprio(3);
          else if (pr == 2) __builtin_amdgcn_s_setprio(2);
          else if (pr == 1) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        }
        consume(buf[st], tt, lo);
      }
    }
  };
  tile_loop(std::integral_constant<bool, kResidualTile>{});
  bool deep = false;
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    deep = deep || (smin[vb] != __builtin_inff() && smin[vb] - m_ref[vb] < kTailLog);
    l_part[vb] += __shfl_xor(l_part[vb], 16);
    l_part[vb] += __shfl_xor(l_part[vb], 32);
  }
  {
    const bool dw = __any(deep);
    if (lane == 0) {
      s_flag[wave] = dw ? 1 : 0;
      s_flag[W + wave] = fold ? 1 : 0;
    }
  }
  __syncthreads();
  {
    // robust numerics: a CTA-uniform decision over the four KV heads
    bool fp32 = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const bool armed = s_flag[w] != 0 &&
                         value_bound<CT, VD>(a, sc[w], s_vs[w], lane) * (float)(p1 - p0) >= kTailArm;
      fp32 |= s_flag[W + w] != 0 || armed;
    }
    if (fp32) {
      // s_q is free: it holds the FP32 path's per-wave scratch; the per-tensor
      // scales are the same for every KV head (sc[0]) and the per-channel
      // value scales come from s_vs
      static_assert(W * (VD + 2) * 4 <= (int)sizeof(s_q), "FP32-path scratch fits the query stage");
#pragma unroll 1
      for (int u = 0; u < W * VB; ++u)
        exact_partial<CT, D, VD, false, false, W, EXT, MT>(a, unit_of(u / VB, u % VB), p0, p1, sc[0],
                                                           s_vs[u / VB],
                                                           reinterpret_cast<float*>(&s_q[0][0]));
      return;
    }
  }

  // ---- this wave's partials, straight from registers: lane (li, lj) holds
  // channels (4 lj + q) CPL + ct of slot li of each head block
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    if (li >= min(16, vgroup - 16 * vb)) continue;
    const HeadSlot hs = head_slot<MT>(a, unit_of(wave, vb), li);
    const int h = hs.h;
    const size_t pair = hs.pair;
    const size_t pidx = pair * S + split;
    Final fin{0.0f, kNegInf};
    if (a.direct) {
      fin = final_of(a, h, m_ref[vb], l_part[vb]);
      if (a.lse_out && lj == 0) a.lse_out[pair] = fin.lse;
    } else if (lj == 0) {
      reinterpret_cast<float2*>(a.ws_ml)[pidx] = make_float2(m_ref[vb], l_part[vb]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int c4 = 0; c4 < C::CPL; c4 += 4) {
        const int ch = (4 * lj + q) * C::CPL + c4;
        float4 o = make_float4(acc[vb][c4][q], acc[vb][c4 + 1][q], acc[vb][c4 + 2][q], acc[vb][c4 + 3][q]);
        o.x *= a.v_mult * v_scale_of(a, sc[0], s_vs[wave], ch);
        o.y *= a.v_mult * v_scale_of(a, sc[0], s_vs[wave], ch + 1);
        o.z *= a.v_mult * v_scale_of(a, sc[0], s_vs[wave], ch + 2);
        o.w *= a.v_mult * v_scale_of(a, sc[0], s_vs[wave], ch + 3);
        if (a.direct)
          store_final<VD>(a, pair, ch, o, fin.f);
        else
          *reinterpret_cast<float4*>(a.ws_acc + pidx * VD + ch) = o;
      }
    }
  }
}

// ---- the latent (absorbed-MLA) kernel -------------------------------------
//
// One cache row per token supplies K (all 576 channels) and V (its first 512
// channels).  A CTA holds G groups of W = 4 waves (built with G = 1: one
// wave per SIMD; with G = 2 every SIMD would run two waves, each group
// taking its own run of W tiles of a round) and walks its position range in
// rounds of G W 16-token tiles.  Tiles are fetched two rounds ahead: with
// one-byte codes on dense rows straight into an LDS ring of four rounds
// (direct-to-LDS loads, see LatCfg::DMA), otherwise into registers.  In a
// round, wave w of a group
//   * computes the scores S^T = K Q'^T of tile w and publishes the tile's
//     maximum per head in LDS,
//   * (register path) copies the tile's raw codes into the round's LDS
//     stage (64 rows),
//   * takes the group's maximum over the W tile maxima (so the group's waves
//     hold the same running reference maximum), turns its own tile's scores
//     into probabilities and publishes them in LDS, and
//   * accumulates V channels [512 w / W, 512 (w + 1) / W) of the group's
//     tokens, reading the V^T operands from the ring or the stage with the
//     LDS transpose reads and the probabilities of all W tiles.
// Each wave evaluates the exponentials of its own tile only; the running
// sums of a group's waves are added at the end.
// Each row therefore crosses HBM and L2 once, V needs no registers while in
// flight, and each wave keeps a 16 x (512 / W) accumulator.  With G > 1 the
// groups' states (m, l, accumulator) are merged in LDS at the end, in group
// order.  Stage and ring rows are padded to keep LDS bank conflicts low.

template <int N>
using ic = std::integral_constant<int, N>;

template <int CT, bool GATHER>
struct LatCfg {
  static constexpr int D = 576, VD = 512;
  static constexpr int EB = (CT == PKV_F16) ? 2 : 1;
  static constexpr int KROW = D * EB;
  static constexpr int NKS = D / 32;
  static constexpr int NKL = KROW / 64;          // 16-byte K loads per lane per tile
  static constexpr int NKW = NKL * 4;
  static constexpr int W = EB == 1 ? kLatentWaves : kWaves;  // waves per group
  static constexpr int G = EB == 1 ? kLatentGroups : 1;      // groups per CTA
  static constexpr int NW = W * G;               // waves per CTA
  static constexpr int NT = 64 * NW;             // threads per CTA
  static constexpr int VQ = VD / W;              // V channels per wave
  static constexpr int CPL = VQ / 16;            // 16-channel column tiles per wave
  // LDS stage row stride (bytes).  One-byte codes: 592 = 148 dwords, which
  // keeps the 16-byte row writes (16 rows x 64 bytes per instruction) free
  // of conflicts on gfx950's 64 LDS banks and leaves the transposed V reads
  // two-way conflicted at most (SQ_LDS_BANK_CONFLICT on the latent FP8
  // workload: 2.6e5 against 8.5e5 with a 608-byte stride).
  static constexpr int RS = KROW + (EB == 1 ? 16 : 64);
  static constexpr int ROUND = 16 * W;          // tokens per group and round
  // one CTA per CU, G waves per SIMD
  static constexpr int MIN_WAVES = G;
  // one group: the folded query stays in registers (one-byte codes); two
  // groups read it from LDS in every round (the registers go to the second
  // wave per SIMD)
  static constexpr bool QREG = EB == 1 && (G == 1 || !GATHER);
  // one-byte codes, dense rows, one group: K tiles go straight to an LDS
  // ring of NSLOT rounds (no register holds K in flight, no stage copy);
  // a tile is NKL 1 KB blocks (block s: lane i's 16 bytes = chunk
  // (i >> 4) + 4 s of token i & 15), padded so that the two tiles of a
  // pair start 32 banks apart for the transposed V reads
  static constexpr bool DMA = EB == 1 && !GATHER && G <= 2;
  static constexpr int NSLOT = 4;
  static constexpr int TB = NKL * 1024 + 128;     // bytes per tile in the ring
  static constexpr int STAGE_BYTES = DMA ? NSLOT * W * TB : G * ROUND * RS;
  static_assert(RS % 16 == 0, "stage rows hold 16-byte chunks");
};

template <class C>
struct LatK {
  uint32_t k[C::NKW];
  uint32_t mask;  // bit q: token 4 lj + q of the tile valid
  bool row_ok;    // token li of the tile valid
};

// LDS transpose reads (gfx950): within each group of 16 lanes, the 8-byte
// pieces the lanes point at form a byte (tr8) or half (tr16) matrix whose
// rows are the pieces of lanes {2k, 2k+1} (tr8: 8 rows of 16 bytes) or
// {4k .. 4k+3} (tr16: 4 rows of 16 halves); lane i of the group receives
// column i -- one element of each row, in row order.
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v2i32 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i32*)p);
}

__device__ __forceinline__ half4 lds_read_tr16(const uint8_t* p) {
  return __builtin_bit_cast(
      half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p));
}

template <int CT, bool GATHER, bool EXT>
__global__ void __launch_bounds__((LatCfg<CT, GATHER>::NT))
__attribute__((amdgpu_waves_per_eu(LatCfg<CT, GATHER>::MIN_WAVES)))
latent_kernel(const SplitArgs a) {
  using C = LatCfg<CT, GATHER>;
  constexpr int W = C::W;
  constexpr int NW = C::NW;
  constexpr int NT = C::NT;
  constexpr int D = C::D;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = C::G == 1 ? 0 : wave / W;  // group
  const int wv = wave - grp * W;    // wave within the group
  const int li = lane & 15;
  const int lj = lane >> 4;
  const int S = a.num_splits;
  const int KVH = a.kv_heads;

  // ---- prologue: every independent read is issued before the first wait
  const bool balanced = a.target_ctas > 0;
  Work wk;
  int raw_npos = 0, raw_len = 0;
  if (balanced) {
    if (!locate_balanced<GATHER, EXT>(a, lane, wk)) return;  // padding CTA
  } else {
    static_item(a, wk);
    raw_npos = GATHER ? uniform_load(a.num_candidates, wk.r) : uniform_load(a.seq_lens, wk.r);
  }
  if constexpr (GATHER) raw_len = uniform_load(a.seq_lens, wk.r);
  unit_heads(a, wk);
  const int r = wk.r, g = wk.g, h0 = wk.h0, nh = wk.nh;

  // DMA ring: Q' and its folding errors live in the last slot until the
  // prologue is over (that slot's first loads go out in the second round)
  __shared__ uint4 s_q_own[C::DMA ? 1 : C::NKS * 64];
  __shared__ float s_err_own[C::DMA ? 1 : C::NKS * 64];  // folding error per Q' entry
  __shared__ int s_flag[NW + 1];                  // per wave: a deep-tail probability; [NW]: folding
  static_assert(W == 4, "one float4 of tile maxima per head");
  __shared__ f32x4 s_tmax[C::G][16];              // per group and head: the round's W tile maxima
  __shared__ half4 s_p[NW][64];                   // per wave: FP16(16 p) of its tile
  __shared__ half4 s_pl[kResidualTile ? NW : 1][64];  // and its residual
  __shared__ float s_lw[NW][16];                  // per wave and head: its running sum
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[C::STAGE_BYTES];
  static_assert(!C::DMA || C::NKS * 64 * 20 <= W * C::TB, "Q' fits a ring slot");
  uint4* const s_q = C::DMA ? reinterpret_cast<uint4*>(s_stage + (C::NSLOT - 1) * W * C::TB) : s_q_own;
  float* const s_err = C::DMA ? reinterpret_cast<float*>(s_stage + (C::NSLOT - 1) * W * C::TB + C::NKS * 64 * 16)
                              : s_err_own;
  __shared__ float s_ml[C::G][16];                // per group: reference maximum per head
  __shared__ float s_vs[C::VD];
  constexpr int QPT = (C::NKS * 64 + NT - 1) / NT;
  uint4 qraw[QPT];
  float4 ksc[QPT][2];
  const int32_t* bt_row = a.block_table + (size_t)r * a.max_blocks_per_row;
  // block ids of this wave's first 64 tiles (static mode: before the length;
  // read again below when a sliding window moves the row's first token)
  WaveBlocks wb{bt_row, wk.base + split_p0(a, wk), wave, NW, 0, 0};
  if constexpr (!GATHER) wb.load(a, 0, lane);
  q_issue<C::NKS, C::EB, D, QPT, NT, false, false>(a, wk, qraw, ksc);
  const Scales sc = load_scales<C::VD, NT>(a, g);
  finish_item<GATHER, EXT>(a, wk, balanced, raw_npos, raw_len);
  const int len = wk.len;
  if constexpr (!GATHER && EXT)
    if (!balanced && wk.base > 0) {
      wb.p0 = wk.base + split_p0(a, wk);
      wb.load(a, 0, lane);
    }
  const int skip = wk.lo - wk.base;  // positions of the row before its window start
  const int base = wk.base;
  const int lo = wk.lo;

  int p0, p1;
  if (!split_range<C::VD, NT>(a, wk, p0, p1)) return;
  const int split = wk.split;
  const int ntiles = (p1 - p0 + 15) >> 4;
  const int nrounds = (ntiles + NW - 1) / NW;

  const uint32_t tok = (uint32_t)KVH * C::KROW;  // bytes per token slot
  const uint32_t koff = (uint32_t)li * tok + (uint32_t)g * C::KROW + 16u * lj;

  // ring address of block s of tile t (round t / NW, this wave's tile)
  const uint32_t ring = lds_addr(s_stage);
  auto dma_dst = [&](int t, int s) __attribute__((always_inline)) {
    const int slot = ((t / NW) * C::G + grp) & (C::NSLOT - 1);
    return (uint32_t)__builtin_amdgcn_readfirstlane(ring + (uint32_t)((slot * W + wv) * C::TB + 1024 * s));
  };
  auto issue_k = [&](LatK<C>& T, int t, auto s0c, auto s1c) __attribute__((always_inline)) {
    constexpr int S0 = decltype(s0c)::value, S1 = decltype(s1c)::value;
    uint32_t m = 0;
    if constexpr (!GATHER) {
      int64_t s0 = 0;
      bool bv = false;
      if (t < ntiles) {
        const int tp = p0 + 16 * t;
        const int blk = wb.of(a, t, lane);
        bv = blk >= 0 && blk < a.num_pool_blocks;
        s0 = bv ? ((int64_t)blk << a.log2_block) + ((base + tp) & (a.block_size - 1)) : 0;
      }
      // the descriptor covers the tile's valid rows only: rows past the end
      // (and a whole tile with an invalid block) read as zeros; so do rows
      // before a sliding window's start (an offset past the descriptor)
      const int tp = p0 + 16 * t;
      const uint32_t nv = bv ? (uint32_t)min(16, p1 - tp) : 0u;
      const auto rs = make_rsrc(a.key_cache + s0 * tok, nv * tok);
      if (EXT && tp < skip) {
        // the row's first tile under a sliding window: rows before the
        // window start read past the descriptor (zeros) and are masked
        const int sk = skip - tp;
        const uint32_t past = li < sk ? kPastDescriptor : 0u;
#pragma unroll
        for (int s = S0; s < S1; ++s) {
          if constexpr (C::DMA)
            buffer_load_lds16(dma_dst(t, s), koff + 64 * s + past, rsrc_words(a.key_cache + s0 * tok, nv * tok));
          else
            buffer_bytes<16>(rs, koff + 64 * s + past, 0, &T.k[4 * s]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * lj + q;
          m |= (row < (int)nv && row >= sk) ? (1u << q) : 0u;
        }
      } else {
#pragma unroll
        for (int s = S0; s < S1; ++s) {
          if constexpr (C::DMA)
            buffer_load_lds16(dma_dst(t, s), koff + 64 * s, rsrc_words(a.key_cache + s0 * tok, nv * tok));
          else
            buffer_bytes<16>(rs, koff + 64 * s, 0, &T.k[4 * s]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) m |= (4 * lj + q < (int)nv) ? (1u << q) : 0u;
      }
      T.row_ok = true;
    } else {
      // per-token slots; invalid entries (and tiles past the end) read token
      // slot 0 of the pool and are masked
      const int pos = p0 + 16 * t + li;
      const int c = (t < ntiles && pos < p1) ? a.candidates[(size_t)r * a.max_candidates + pos] : -1;
      bool v = c >= lo && c < len;
      const int blk = v ? bt_row[c >> a.log2_block] : 0;
      v = v && blk >= 0 && blk < a.num_pool_blocks;
      const int64_t sl = v ? ((int64_t)blk << a.log2_block) + (c & (a.block_size - 1)) : 0;
      const uint8_t* krow = a.key_cache + ((size_t)sl * KVH + g) * C::KROW;
#pragma unroll
      for (int s = S0; s < S1; ++s) load_bytes<16>(krow + 64 * s + 16 * lj, &T.k[4 * s]);
      const int vi = v ? 1 : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) m |= __shfl(vi, 4 * lj + q) ? (1u << q) : 0u;
      T.row_ok = v;
    }
    T.mask = m;
  };

  f32x4 acc[C::CPL];
#pragma unroll
  for (int ct = 0; ct < C::CPL; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;
  float l_part = 0.0f;
  float smin = __builtin_inff();  // smallest valid score of this wave's tiles (lane's head)

  // this lane's 16-byte K chunks of its tile row in the group's stage
  uint8_t* const stage_g = s_stage + (size_t)grp * C::ROUND * C::RS;
  uint8_t* const stage_k = stage_g + (size_t)(16 * wv + li) * C::RS + 16 * lj;
  // the piece this lane contributes to a transposed V read (see lds_read_tr8
  // / lds_read_tr16): one-byte codes -- row k = li / 2 of k-group lj is token
  // 4 lj + (k & 3) of the first (k < 4) or second tile of a tile pair, bytes
  // [8 (li & 1), +8) of a 16-channel column tile; two-byte codes -- row
  // k = li / 4 is token 4 lj + k of a tile, halves [4 (li & 3), +4).
  const uint8_t* stage_v;
  if constexpr (C::EB == 1)
    stage_v = stage_g + (size_t)(16 * ((li >> 1) >> 2) + 4 * lj + ((li >> 1) & 3)) * C::RS +
              (size_t)wv * C::VQ + 8 * (li & 1);
  else
    stage_v = stage_g + (size_t)(4 * lj + (li >> 2)) * C::RS + (size_t)(wv * C::VQ + 4 * (li & 3)) * 2;
  // the same piece in the DMA ring: row k = li / 2 is token 4 lj + (k & 3) of
  // tile (k >> 2) of the pair; this wave's channel chunks 8 wv .. 8 wv + 7 are
  // blocks 2 wv, 2 wv + 1 of the tile, lane slots token + 16 (chunk & 3)
  const uint8_t* const ring_v = s_stage + (size_t)((li >> 1) >> 2) * C::TB + 2048 * wv +
                                16 * (4 * lj + ((li >> 1) & 3)) + 8 * (li & 1);

  // Round rd on the K tile in T.  One-byte codes: the loads of round
  // rd + kAhead go into the buffer Tn (for the mask; with the ring the data
  // goes to its slot), the first kFirstLoads of them before anything else
  // and the rest after the first barrier, so that the four waves' load
  // bursts do not stall their issue for the whole round (measured faster
  // than one burst, and than waiting for T); two-byte codes (whose tiles
  // are twice as large) issue them into T once it is staged.
  constexpr bool kEarly = C::EB == 1;
  // Rounds of lead.  Register path: two.  LDS ring: one -- on C5-shaped
  // work a ring one round ahead measured faster than two (21.4-21.9 against
  // 22.3-22.9 us) and three slower still (24.6): more outstanding loads per
  // CU only lengthen their latency -- with three of the nine loads issued
  // at the round start and six after the first barrier (all nine after it:
  // 26.2 us; five or seven first: 21.8, 22.0).  Two groups on the ring hold
  // exactly the current and the next 128-token round in the four slots, so
  // there all nine loads wait for the first barrier (every wave past the
  // previous round's V reads).
  constexpr int kAhead = C::DMA ? 1 : 2;
  constexpr int kFirstLoads = (C::DMA && C::G > 1) ? 0 : (C::DMA ? 3 : (C::NKL + 1) / 2);
  // one group, one-byte codes: Q' is read from LDS into registers once
  half8 qreg[C::QREG ? C::NKS : 1];
  auto round = [&](LatK<C>& T, LatK<C>& Tn, int rd, auto lo) __attribute__((always_inline)) {
    constexpr bool LO = decltype(lo)::value;
    if constexpr (kEarly) issue_k(Tn, (rd + kAhead) * NW + wave, ic<0>{}, ic<kFirstLoads>{});
    // keep the loads ahead of the waits for this round's data
    __builtin_amdgcn_sched_barrier(0);
    const int slot = (rd * C::G + grp) & (C::NSLOT - 1);
    if constexpr (C::DMA) {
      // this round's tile has landed once only the next round's loads and
      // the first part of round rd + 2's are outstanding
      wait_vmcnt<(kAhead - 1) * C::NKL + kFirstLoads>();
      const uint8_t* tile = s_stage + (size_t)(slot * W + wv) * C::TB + 16 * lane;
#pragma unroll
      for (int s = 0; s < C::NKL; ++s) {
        const uint4 u = *reinterpret_cast<const uint4*>(tile + 1024 * s);
        T.k[4 * s] = u.x;
        T.k[4 * s + 1] = u.y;
        T.k[4 * s + 2] = u.z;
        T.k[4 * s + 3] = u.w;
      }
    }
    // scores of this wave's tile
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::NKL; ++s) {
      if constexpr (C::EB == 2) {
        const half8 kop = __builtin_bit_cast(
            half8, uint4{T.k[4 * s], T.k[4 * s + 1], T.k[4 * s + 2], T.k[4 * s + 3]});
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, __builtin_bit_cast(half8, s_q[s * 64 + lane]), sacc, 0, 0, 0);
      } else {
        const half4 c0 = codes4_to_half4<CT>(T.k[4 * s + 0]);
        const half4 c1 = codes4_to_half4<CT>(T.k[4 * s + 1]);
        const half4 c2 = codes4_to_half4<CT>(T.k[4 * s + 2]);
        const half4 c3 = codes4_to_half4<CT>(T.k[4 * s + 3]);
        const half8 k0 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const half8 k1 = {c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
        if constexpr (C::QREG) {
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qreg[2 * s], sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qreg[2 * s + 1], sacc, 0, 0, 0);
        } else {
          const half8 q0 = __builtin_bit_cast(half8, s_q[(2 * s) * 64 + lane]);
          const half8 q1 = __builtin_bit_cast(half8, s_q[(2 * s + 1) * 64 + lane]);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q0, sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q1, sacc, 0, 0, 0);
        }
      }
    }
    float scw[4];
    float xs[4];
    scaled_scores<EXT>(a, sacc, xs);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool valid = (T.mask >> q) & 1u;
      scw[q] = valid ? xs[q] : kNegInf;
      smin = fminf(smin, valid ? scw[q] : __builtin_inff());
    }
    // the tile's maximum per head (lanes li, li + 16, li + 32, li + 48)
    float tm = fmaxf(fmaxf(scw[0], scw[1]), fmaxf(scw[2], scw[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    if (lj == 0) reinterpret_cast<float*>(&s_tmax[grp][li])[wv] = tm;
    // every wave is past the previous round's V and probability reads and
    // has published its tile maximum (single buffers suffice: a wave reads
    // the maxima, the stage and the probabilities of round rd before the
    // first barrier of round rd + 1, and they are next written after it)
    __syncthreads();
    if constexpr (kEarly) issue_k(Tn, (rd + kAhead) * NW + wave, ic<kFirstLoads>{}, ic<C::NKL>{});
    // invalid rows are stored as zeros, so the V operands need no mask
    // (dense rows: already zero from the buffer descriptor)
    if constexpr (!C::DMA) {
      const uint32_t keep = (GATHER && !T.row_ok) ? 0u : 0xffffffffu;
#pragma unroll
      for (int s = 0; s < C::NKL; ++s)
        *reinterpret_cast<uint4*>(stage_k + 64 * s) =
            uint4{T.k[4 * s] & keep, T.k[4 * s + 1] & keep, T.k[4 * s + 2] & keep, T.k[4 * s + 3] & keep};
    }
    if constexpr (!kEarly) issue_k(T, (rd + 2) * NW + wave, ic<0>{}, ic<C::NKL>{});
    __builtin_amdgcn_sched_barrier(0);

    const f32x4 tmx = s_tmax[grp][li];
    const float mt = fmaxf(fmaxf(tmx[0], tmx[1]), fmaxf(tmx[2], tmx[3]));
    if (__any(mt > m_ref + kRescaleSlack)) {
      const float mn = fmaxf(m_ref, mt);
      const float alpha = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - mn) * kLog2e);
      l_part *= alpha;
#pragma unroll
      for (int ct = 0; ct < C::CPL; ++ct) acc[ct] *= alpha;
      m_ref = mn;
    }
    const float mu = (m_ref == kNegInf) ? 0.0f : m_ref;
    {
      float p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = __builtin_amdgcn_exp2f((scw[q] - mu) * kLog2e);
      l_part += (p[0] + p[1]) + (p[2] + p[3]);
      half4 po, pr;  // FP16(16 p) and its residual
      split_prob<LO>(p, po, pr);
      s_p[wave][lane] = po;
      if constexpr (LO) s_pl[wave][lane] = pr;
    }
    // the stage and the probabilities hold all 64 rows of the round
    __syncthreads();
    if constexpr (C::EB == 1) {
      // O^T += V^T P^T over tile pairs with 16x16x32 MFMAs: k index 8 lj + e
      // is token 4 lj + (e & 3) of tile 2 m + (e >> 2), in both operands
#pragma unroll
      for (int m = 0; m < W / 2; ++m) {
        const half4 p0 = s_p[grp * W + 2 * m][lane], p1 = s_p[grp * W + 2 * m + 1][lane];
        const half8 pb = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        half8 pl = {};
        if constexpr (LO) {
          const half4 r0 = s_pl[grp * W + 2 * m][lane], r1 = s_pl[grp * W + 2 * m + 1][lane];
          pl = half8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        }
        // all V^T reads of the tile pair go out before their conversions:
        // one LDS round trip per pair instead of one per column tile
        v2i32 raws[C::CPL];
#pragma unroll
        for (int ct = 0; ct < C::CPL; ++ct) {
          if constexpr (C::DMA)
            raws[ct] = lds_read_tr8(ring_v + (size_t)(slot * W + 2 * m) * C::TB + 1024 * (ct >> 2) + 256 * (ct & 3));
          else
            raws[ct] = lds_read_tr8(stage_v + (size_t)(32 * m) * C::RS + 16 * ct);
        }
#pragma unroll
        for (int ct = 0; ct < C::CPL; ++ct) {
          const v2i32 raw = raws[ct];
          const half4 lo = codes4_to_half4<CT>((uint32_t)raw.x);
          const half4 hi = codes4_to_half4<CT>((uint32_t)raw.y);
          const half8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, acc[ct], 0, 0, 0);
          if constexpr (LO) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl, acc[ct], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const half4 pj = s_p[grp * W + j][lane];
        half4 rj = {};
        if constexpr (LO) rj = s_pl[grp * W + j][lane];
#pragma unroll
        for (int ct = 0; ct < C::CPL; ++ct) {
          const half4 va = lds_read_tr16(stage_v + (size_t)(16 * j) * C::RS + 32 * ct);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pj, acc[ct], 0, 0, 0);
          if constexpr (LO) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, rj, acc[ct], 0, 0, 0);
        }
      }
    }
  };

  // kAhead rounds of K in flight (deeper rings measured slower on MI355X:
  // more outstanding misses per CU only lengthen the latency)
  LatK<C> ka, kb, kc;
  issue_k(ka, wave, ic<0>{}, ic<C::NKL>{});
  if constexpr (kAhead == 2) issue_k(kb, NW + wave, ic<0>{}, ic<C::NKL>{});
  q_stage<C::NKS, C::EB, D, QPT, NT>(qraw, ksc, sc.k_tensor, s_q, s_err);
  stage_scales<C::VD, NT>(a, sc, s_vs);
  __syncthreads();
  // folding bound of the CTA's heads (read after the final barrier)
  if (wave == 0) {
    const bool fold = fold_over_budget<CT, C::NKS>(a, s_err, nh, lane);
    if (lane == 0) s_flag[NW] = fold ? 1 : 0;
  }
  if constexpr (C::QREG) {
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) qreg[s] = __builtin_bit_cast(half8, s_q[s * 64 + lane]);
  }
  auto round_loop = [&](auto lo) __attribute__((always_inline)) {
    if constexpr (kEarly && kAhead == 1) {
      for (int rd = 0; rd < nrounds; rd += 3) {
        round(ka, kb, rd, lo);
        if (rd + 1 >= nrounds) break;
        round(kb, kc, rd + 1, lo);
        if (rd + 2 >= nrounds) break;
        round(kc, ka, rd + 2, lo);
      }
    } else if constexpr (kEarly) {
      for (int rd = 0; rd < nrounds; rd += 3) {
        round(ka, kc, rd, lo);
        if (rd + 1 >= nrounds) break;
        round(kb, ka, rd + 1, lo);
        if (rd + 2 >= nrounds) break;
        round(kc, kb, rd + 2, lo);
      }
    } else {
      for (int rd = 0; rd < nrounds; rd += 2) {
        round(ka, ka, rd, lo);
        if (rd + 1 >= nrounds) break;
        round(kb, kb, rd + 1, lo);
      }
    }
  };
  round_loop(std::integral_constant<bool, kResidualTile>{});
  // the ring's last loads (rounds past the end, zero-filled) land before
  // the LDS is used again
  if constexpr (C::DMA) wait_vmcnt<0>();
  // every wave of a group holds the group's running maximum and the sum over
  // its own tiles: sum the lane groups, then the group's waves in order; the
  // CTA's reference maximum is the largest of the groups'
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
  if (lj == 0) s_lw[wave][li] = l_part;
  if (C::G > 1 && wv == 0 && lane < 16) s_ml[grp][lane] = m_ref;
  __syncthreads();
  l_part = 0.0f;
#pragma unroll
  for (int j = 0; j < W; ++j) l_part += s_lw[grp * W + j][li];
  float m_all = m_ref;
  if constexpr (C::G > 1) {
#pragma unroll
    for (int j = 0; j < C::G; ++j) m_all = fmaxf(m_all, s_ml[j][li]);
  }
  // a valid probability that fell below the FP16 tile's normal range: some
  // score more than ln 2^18 below the final reference maximum (conservative)
  const bool deep = smin != __builtin_inff() && smin - m_all < kTailLog;

  {
    const bool dw = __any(deep);
    if (lane == 0) s_flag[wave] = dw ? 1 : 0;
  }
  __syncthreads();
  {
    // robust numerics: recompute on the FP32 path when the folding bound or
    // the tail-depth check fails (a CTA-uniform decision); the stage is free
    bool deep_any = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) deep_any |= s_flag[w] != 0;
    const bool armed = deep_any && value_bound<CT, C::VD>(a, sc, s_vs, lane) * (float)(p1 - p0) >= kTailArm;
    if (s_flag[NW] != 0 || (deep_any && armed)) {
      static_assert(NW * (C::VD + 2) * 4 <= C::G * C::ROUND * C::RS, "FP32-path scratch fits the stage");
      exact_partial<CT, D, C::VD, true, GATHER, NW, EXT>(a, wk, p0, p1, sc, s_vs,
                                                    reinterpret_cast<float*>(s_stage));
      return;
    }
  }

  if constexpr (C::G > 1) {
    // groups 1 .. G-1 hand their accumulators to group 0 through the stage
    // (free: every wave is past its last V read), which merges them in group
    // order with the weights exp(m_j - m_all)
    static_assert((C::G - 1) * W * C::CPL * 64 * 16 <= C::G * C::ROUND * C::RS, "accumulators fit the stage");
    f32x4* const xacc = reinterpret_cast<f32x4*>(s_stage);
    if (grp > 0) {
#pragma unroll
      for (int ct = 0; ct < C::CPL; ++ct) xacc[(((grp - 1) * W + wv) * C::CPL + ct) * 64 + lane] = acc[ct];
    }
    __syncthreads();
    if (grp > 0) return;
    const float f0 = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_all) * kLog2e);
    l_part *= f0;
#pragma unroll
    for (int ct = 0; ct < C::CPL; ++ct) acc[ct] *= f0;
#pragma unroll
    for (int j = 1; j < C::G; ++j) {
      const float mj = s_ml[j][li];
      const float fj = (mj == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((mj - m_all) * kLog2e);
      float lj_sum = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) lj_sum += s_lw[j * W + w][li];
      l_part += fj * lj_sum;
#pragma unroll
      for (int ct = 0; ct < C::CPL; ++ct) acc[ct] += fj * xacc[(((j - 1) * W + wv) * C::CPL + ct) * 64 + lane];
    }
    m_ref = m_all;
  }
  if (li < nh) {
    const int h = h0 + li;
    const size_t pidx = ((size_t)r * a.heads + h) * S + split;
    const size_t pair = (size_t)r * a.heads + h;
    Final fin{0.0f, kNegInf};
    if (a.direct) {
      fin = final_of(a, h, m_ref, l_part);
      if (a.lse_out && wave == 0 && lj == 0) a.lse_out[pair] = fin.lse;
    } else if (wave == 0 && lj == 0) {
      reinterpret_cast<float2*>(a.ws_ml)[pidx] = make_float2(m_ref, l_part);
    }
    float* dst = a.ws_acc + pidx * C::VD;
    // column tile ct holds channels 16 ct + 4 lj + q of this wave's range
#pragma unroll
    for (int ct = 0; ct < C::CPL; ++ct) {
      const int cbase = wv * C::VQ + 16 * ct + 4 * lj;
      float4 o;
      float* op = reinterpret_cast<float*>(&o);
#pragma unroll
      for (int q = 0; q < 4; ++q) op[q] = (acc[ct][q] * a.v_mult) * v_scale_of(a, sc, s_vs, cbase + q);
      if (a.direct)
        store_final<C::VD>(a, pair, cbase, o, fin.f);
      else
        *reinterpret_cast<float4*>(dst + cbase) = o;
    }
  }
}

// ---- the combine kernel ---------------------------------------------------
//
// One CTA per (row, query head).  Wave 0 turns the S (m, l) pairs into merge
// weights w_k = exp(m_k - M) and L = sum_k w_k l_k; then every thread owns one
// float4 of channels and a fixed subset of splits, issues all of its partial
// loads at once, and the per-thread sums are added across the split subsets
// in a fixed order through LDS, so the result does not depend on timing.

// Threads per CTA: 128 for 64 channels (8 split subsets of the 16 float4
// channel groups), 512 for 128 and 512 channels, 1024 for 256 (16 subsets).
// Measured on MI355X: 512 threads at 64 channels -- 32 subsets of two
// splits each and a 32-way reduction -- made the combine of the
// PagedAttention 16384-token x 32-row shape 8.4 us slower; 256 or 1024
// threads at 128 channels were no better; at 256 channels 1024 threads took
// 0.35 us off the single-row INT8 step and 256 added 0.6.
template <int VD>
constexpr int combine_threads() { return VD == 64 ? 128 : (VD == 256 ? 1024 : 512); }

template <int VD, bool OUT_F32>
__global__ void __launch_bounds__(combine_threads<VD>())
combine_kernel(const CombineArgs a) {
  constexpr int CG = VD / 4;                  // float4 channel groups
  constexpr int KS = combine_threads<VD>() / CG;  // split subsets
  constexpr int MAXI = (kMaxSplits + KS - 1) / KS;
  const int pair = blockIdx.x;
  const int t = threadIdx.x;
  const int cg = t % CG;
  const int ks = t / CG;
  const int h = pair % a.heads;
  const int S = a.num_splits;

  __shared__ float s_w[kMaxSplits];
  __shared__ float s_ml[2];
  __shared__ float4 s_part[KS][CG];

  if (t < 64) {
    float mk = kNegInf, lk = 0.0f;
    if (t < S) {
      const float2 v = reinterpret_cast<const float2*>(a.ws_ml)[(size_t)pair * S + t];
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
    if (t < kMaxSplits) s_w[t] = w;
    if (t == 0) {
      s_ml[0] = M;
      s_ml[1] = L;
    }
  }

  // Partial loads are issued before the weights are known (an empty split's
  // accumulator is read and ignored) -- for every split in the static
  // decomposition, and for the first kSpecSplits in the live-balanced one,
  // where most of the S slots of a short row can be empty; there the later
  // slots are read only when their weight is nonzero.
  constexpr int kSpecSplits = 16;
  const int spec = a.skip_empty ? min(S, kSpecSplits) : S;
  const float* base = a.ws_acc + (size_t)pair * S * VD + cg * 4;
  float4 v[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int k = ks + i * KS;
    if (k < spec) v[i] = *reinterpret_cast<const float4*>(base + (size_t)k * VD);
  }
  __syncthreads();
  if (spec < S) {
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int k = ks + i * KS;
      if (k >= spec && k < S && s_w[k] != 0.0f)
        v[i] = *reinterpret_cast<const float4*>(base + (size_t)k * VD);
    }
  }
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int k = ks + i * KS;
    if (k < S) {
      const float w = s_w[k];
      if (w != 0.0f) {  // empty splits' accumulators are never used
        o.x += w * v[i].x;
        o.y += w * v[i].y;
        o.z += w * v[i].z;
        o.w += w * v[i].w;
      }
    }
  }
  s_part[ks][cg] = o;
  __syncthreads();
  if (ks != 0) return;
  float4 r = s_part[0][cg];
#pragma unroll
  for (int j = 1; j < KS; ++j) {
    const float4 q = s_part[j][cg];
    r.x += q.x;
    r.y += q.y;
    r.z += q.z;
    r.w += q.w;
  }
  const float M = s_ml[0], L = s_ml[1];
  float lse = kNegInf;
  float f = 0.0f;
  if (L > 0.0f) {
    lse = M + logf(L);
    f = 1.0f / L;
    if (a.head_sink) f *= 1.0f / (1.0f + expf(a.head_sink[h] - lse));
  }
  if (a.lse_out && t == 0) a.lse_out[pair] = lse;
  if constexpr (OUT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + (size_t)pair * VD + cg * 4) =
        make_float4(r.x * f, r.y * f, r.z * f, r.w * f);
  } else {
    const half4 hv = {(half_t)(r.x * f), (half_t)(r.y * f), (half_t)(r.z * f), (half_t)(r.w * f)};
    *reinterpret_cast<half4*>(reinterpret_cast<half_t*>(a.out) + (size_t)pair * VD + cg * 4) = hv;
  }
}

// ---- the combine for few splits -------------------------------------------
//
// For few splits (S <= 8): PARTS waves per (row, query head), each owning
// VD / PARTS channels (PARTS = 2 for 512 channels, so every lane loads one
// float4 per split and twice as many CUs pull the partials), four waves per
// CTA, so a step with many rows does not launch one 512-thread CTA per
// pair.  The (m, l) pairs are
// wave-uniform and come through scalar loads; every lane owns VD / 64 /
// PARTS consecutive channels, issues all of its partial loads first and sums
// the weighted partials in split order (deterministic).  Same arithmetic as
// combine_kernel, so S = 1 gives what the kernels' direct output gives.

template <int VD, bool OUT_F32, int kSmallSplits, int PARTS>
__global__ void __launch_bounds__(256) combine_small_kernel(const CombineArgs a) {
  constexpr int CPL = VD / 64 / PARTS;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * 4 + wave;
  const int pair = item / PARTS;
  const int part = item - pair * PARTS;
  if (pair >= a.rows * a.heads) return;
  const int S = a.num_splits;
  const int h = pair % a.heads;
  const int c0 = part * (VD / PARTS) + lane * CPL;  // first channel of this lane

  const float* base = a.ws_acc + (size_t)pair * S * VD + c0;
  float v[kSmallSplits][CPL];
#pragma unroll
  for (int k = 0; k < kSmallSplits; ++k) {
    if (k < S) {
      if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < CPL; j += 4) {
          const float4 q = *reinterpret_cast<const float4*>(base + (size_t)k * VD + j);
          v[k][j] = q.x; v[k][j + 1] = q.y; v[k][j + 2] = q.z; v[k][j + 3] = q.w;
        }
      } else if constexpr (CPL == 2) {
        const float2 q = *reinterpret_cast<const float2*>(base + (size_t)k * VD);
        v[k][0] = q.x; v[k][1] = q.y;
      } else {
        v[k][0] = base[(size_t)k * VD];
      }
    }
  }
  float mk[kSmallSplits], lk[kSmallSplits];
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < kSmallSplits; ++k) {
    mk[k] = kNegInf;
    lk[k] = 0.0f;
    if (k < S) {
      mk[k] = uniform_load(a.ws_ml, 2 * ((size_t)pair * S + k));
      lk[k] = uniform_load(a.ws_ml, 2 * ((size_t)pair * S + k) + 1);
    }
    M = fmaxf(M, mk[k]);
  }
  float L = 0.0f;
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < kSmallSplits; ++k) {
    if (k < S) {
      const float w = (mk[k] == kNegInf) ? 0.0f : expf(mk[k] - M);
      L += w * lk[k];
      if (w != 0.0f) {  // empty splits' accumulators are never used
#pragma unroll
        for (int j = 0; j < CPL; ++j) o[j] += w * v[k][j];
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
  if (a.lse_out && lane == 0 && part == 0) a.lse_out[pair] = lse;
  if constexpr (OUT_F32) {
    float* dst = reinterpret_cast<float*>(a.out) + (size_t)pair * VD + c0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) dst[j] = o[j] * f;
  } else {
    half_t* dst = reinterpret_cast<half_t*>(a.out) + (size_t)pair * VD + c0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) dst[j] = (half_t)(o[j] * f);
  }
}

// ---- the wave-per-pair combine for many pairs ------------------------------
//
// One wave per (row, query head) (PARTS waves for 512 channels), four waves
// per CTA, for any S up to 64: lane k reads the (m, l) of split k, the wave
// reduces M and L with butterflies (a fixed order), and n = 1 + the last
// split with a nonzero weight bounds the partial loads -- the splits of a
// row that hold work come first in both decompositions, so a short row of
// the live-balanced decomposition reads only its own few partials.  The
// first SPEC splits are loaded before the weights are known (a slot past n
// is read and ignored), the rest in batches once n is known.  Each lane owns
// VD / 64 / PARTS consecutive channels and adds the weighted partials in
// split order.  With many pairs this keeps every CU busy with small CTAs
// where combine_kernel's one 512-thread CTA per pair runs in several
// dependent rounds.

template <int CPL>
__device__ __forceinline__ void load_channels(const float* p, float (&d)[CPL]) {
  if constexpr (CPL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < CPL; j += 4) {
      const float4 q = *reinterpret_cast<const float4*>(p + j);
      d[j] = q.x; d[j + 1] = q.y; d[j + 2] = q.z; d[j + 3] = q.w;
    }
  } else if constexpr (CPL == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    d[0] = q.x; d[1] = q.y;
  } else {
    d[0] = p[0];
  }
}

template <int VD, bool OUT_F32, int PARTS, int SPEC>
__global__ void __launch_bounds__(256) combine_wave_kernel(const CombineArgs a) {
  constexpr int CPL = VD / 64 / PARTS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * 4 + wave;
  const int pair = item / PARTS;
  const int part = item - pair * PARTS;
  if (pair >= a.rows * a.heads) return;
  const int S = a.num_splits;
  const int h = pair % a.heads;
  const int c0 = part * (VD / PARTS) + lane * CPL;
  const float* base = a.ws_acc + (size_t)pair * S * VD + c0;
  float v[SPEC > 0 ? SPEC : 1][CPL];
#pragma unroll
  for (int k = 0; k < SPEC; ++k)
    if (k < S) load_channels<CPL>(base + (size_t)k * VD, v[k]);
  float mk = kNegInf, lk = 0.0f;
  if (lane < S) {
    const float2 q = reinterpret_cast<const float2*>(a.ws_ml)[(size_t)pair * S + lane];
    mk = q.x;
    lk = q.y;
  }
  float M = mk;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float w = (mk == kNegInf) ? 0.0f : expf(mk - M);
  float L = w * lk;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
  const uint64_t nz = __ballot(w != 0.0f);
  const int n = nz ? 64 - __builtin_clzll(nz) : 0;
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < SPEC; ++k) {
    if (k < n) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
      if (wk != 0.0f) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) o[j] += wk * v[k][j];
      }
    }
  }
  constexpr int NB = CPL <= 2 ? 32 : 16;  // partial loads per batch
  for (int k0 = SPEC; k0 < n; k0 += NB) {
    float u[NB][CPL];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (k0 + i < n) load_channels<CPL>(base + (size_t)(k0 + i) * VD, u[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (k0 + i < n) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k0 + i));
        if (wk != 0.0f) {
#pragma unroll
          for (int j = 0; j < CPL; ++j) o[j] += wk * u[i][j];
        }
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
  if (a.lse_out && lane == 0 && part == 0) a.lse_out[pair] = lse;
  if constexpr (OUT_F32) {
    float* dst = reinterpret_cast<float*>(a.out) + (size_t)pair * VD + c0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) dst[j] = o[j] * f;
  } else {
    half_t* dst = reinterpret_cast<half_t*>(a.out) + (size_t)pair * VD + c0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) dst[j] = (half_t)(o[j] * f);
  }
}

// ---- dispatch ---------------------------------------------------------------

template <int CT, int D, int VD, bool LAT, bool GA, bool EXT, bool MT>
static hipError_t launch_one(const SplitArgs& a, hipStream_t stream) {
  dim3 grid(a.grid_ctas);
  if constexpr (MT && (LAT || GA)) {
    return hipErrorInvalidValue;  // several tokens per row: dense rows, separate caches
  } else {
    if constexpr (!LAT && !GA) {
      const bool two = a.qtok * a.group > 16;  // two head blocks per wave
      if (a.kvp == 4 && !two) {
        hipLaunchKernelGGL((split_kvp_kernel<CT, D, VD, EXT, 4, MT, 1>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
      }
      if constexpr (D <= 128)
        if (a.kvp == 4 && two) {
          hipLaunchKernelGGL((split_kvp_kernel<CT, D, VD, EXT, 4, MT, 2>), grid, dim3(256), 0, stream, a);
          return hipGetLastError();
        }
      if (a.kvp == 8 && !two) {
        hipLaunchKernelGGL((split_kvp_kernel<CT, D, VD, EXT, 8, MT, 1>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
      }
      if (a.kvp) return hipErrorInvalidValue;
    }
    if constexpr (LAT)
      hipLaunchKernelGGL((latent_kernel<CT, GA, EXT>), grid, dim3(LatCfg<CT, GA>::NT), 0, stream, a);
    else
      hipLaunchKernelGGL((split_kernel<CT, D, VD, LAT, GA, EXT, MT>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
}

template <int CT, int D, int VD, bool LAT, bool GA, bool EXT, bool MT>
static hipError_t occupancy_one(int* n, int kvp, int vb) {
  if constexpr (MT && (LAT || GA)) {
    return hipErrorInvalidValue;
  } else {
    if constexpr (!LAT && !GA) {
      if (kvp == 4 && vb == 1)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, split_kvp_kernel<CT, D, VD, EXT, 4, MT, 1>,
                                                             256, 0);
      if constexpr (D <= 128)
        if (kvp == 4 && vb == 2)
          return hipOccupancyMaxActiveBlocksPerMultiprocessor(
              n, split_kvp_kernel<CT, D, VD, EXT, 4, MT, 2>, 256, 0);
      if (kvp == 8 && vb == 1)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, split_kvp_kernel<CT, D, VD, EXT, 8, MT, 1>,
                                                             512, 0);
      if (kvp) return hipErrorInvalidValue;
    }
    if constexpr (LAT)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, latent_kernel<CT, GA, EXT>,
                                                           LatCfg<CT, GA>::NT, 0);
    else
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, split_kernel<CT, D, VD, LAT, GA, EXT, MT>,
                                                           kThreads, 0);
  }
}

// Calls F<CT, D, VD, LAT, GA, EXT, MT>(args...) for the compiled variant;
// returns hipErrorInvalidValue for a variant that is not compiled.  Several
// query tokens per row (MT) are compiled for dense rows of separate caches.
#define PKV_FOR_VARIANT(v, CALL)                                                   \
  do {                                                                             \
    const int hs = (v).head_size, vhs = (v).v_head_size;                           \
    const bool lat = (v).latent != 0, ga = (v).gathered != 0, ext = (v).ext != 0;  \
    const bool mt = (v).mt != 0;                                                   \
    switch ((v).cache_dtype) {                                                     \
      case PKV_F16: PKV_SHAPES(PKV_F16, CALL); break;                              \
      case PKV_I8: PKV_SHAPES(PKV_I8, CALL); break;                                \
      case PKV_FP8_E4M3FN: PKV_SHAPES(PKV_FP8_E4M3FN, CALL); break;                \
      default: break;                                                              \
    }                                                                              \
  } while (0)

#define PKV_MT(CT, D, VD, LAT, GA, EXT, CALL)                                      \
  do {                                                                             \
    if (!mt) { CALL(CT, D, VD, LAT, GA, EXT, false); }                             \
    else if (!LAT && !GA) { CALL(CT, D, VD, LAT, GA, EXT, true); }                 \
  } while (0)

#define PKV_EXT(CT, D, VD, LAT, GA, CALL) \
  do { if (ext) { PKV_MT(CT, D, VD, LAT, GA, true, CALL); } else { PKV_MT(CT, D, VD, LAT, GA, false, CALL); } } while (0)

#define PKV_GATHER(CT, D, VD, LAT, CALL) \
  do { if (ga) { PKV_EXT(CT, D, VD, LAT, true, CALL); } else { PKV_EXT(CT, D, VD, LAT, false, CALL); } } while (0)

#define PKV_SHAPES(CT, CALL)                                                       \
  do {                                                                             \
    if (!lat && hs == 64 && vhs == 64) PKV_GATHER(CT, 64, 64, false, CALL);        \
    else if (!lat && hs == 128 && vhs == 128) PKV_GATHER(CT, 128, 128, false, CALL);\
    else if (!lat && hs == 256 && vhs == 256) PKV_GATHER(CT, 256, 256, false, CALL);\
    else if (lat && hs == 576 && vhs == 512) PKV_GATHER(CT, 576, 512, true, CALL); \
  } while (0)

bool variant_supported(const Variant& v) {
  bool ok = false;
#define PKV_MARK(CT, D, VD, LAT, GA, EXT, MT) ok = true
  PKV_FOR_VARIANT(v, PKV_MARK);
#undef PKV_MARK
  return ok;
}

hipError_t launch_split(const Variant& v, const SplitArgs& a, hipStream_t stream) {
  hipError_t err = hipErrorInvalidValue;
#define PKV_LAUNCH(CT, D, VD, LAT, GA, EXT, MT) err = launch_one<CT, D, VD, LAT, GA, EXT, MT>(a, stream)
  PKV_FOR_VARIANT(v, PKV_LAUNCH);
#undef PKV_LAUNCH
  return err;
}

hipError_t split_occupancy(const Variant& v, int* ctas_per_cu) {
  hipError_t err = hipErrorInvalidValue;
#define PKV_OCC(CT, D, VD, LAT, GA, EXT, MT) err = occupancy_one<CT, D, VD, LAT, GA, EXT, MT>(ctas_per_cu, v.kvp, v.vb)
  PKV_FOR_VARIANT(v, PKV_OCC);
#undef PKV_OCC
  return err;
}

template <int VD, bool F32>
static hipError_t launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  const int pairs = a.rows * a.heads;
  // measured on MI355X: a wave per pair wins up to 8 splits, up to 16 once
  // there are enough pairs to fill the chip with its small CTAs, and for any
  // split count from 1024 pairs (C3 with 8 tokens per row: 4096 pairs, 28
  // splits, step 79.3 -> 70.5 us) with at least 128 channels; with fewer
  // pairs and more splits one CTA per pair pulls its partials in fewer
  // dependent rounds (C2: 64 splits, 6.6 against 8.5 us or more), and at 64
  // channels (one 4-byte load per lane and split) with its 16-byte loads (the
  // 16384 x 32 INT8 page shape: 2048 pairs of 64 full splits, 0.6 us ahead)
  constexpr int PARTS = VD > 256 ? 2 : 1;  // waves per pair
  const int ctas = (pairs * PARTS + 3) / 4;
  if (a.num_splits <= 8)
    hipLaunchKernelGGL((combine_small_kernel<VD, F32, 8, PARTS>), dim3(ctas), dim3(256), 0, stream, a);
  else if (a.num_splits <= 16 && VD <= 256 && pairs >= 512)
    hipLaunchKernelGGL((combine_wave_kernel<VD, F32, PARTS, 16>), dim3(ctas), dim3(256), 0, stream, a);
  else if (pairs >= 1024 && VD >= 128)
    hipLaunchKernelGGL((combine_wave_kernel<VD, F32, PARTS, 8>), dim3(ctas), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<VD, F32>), dim3(pairs), dim3(combine_threads<VD>()), 0, stream, a);
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
