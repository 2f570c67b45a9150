/*
 * pkv.h -- C ABI of libpkv: split-KV (flash-decoding) grouped-query decode
 * attention over a paged KV cache stored as FP16, INT8 or FP8-e4m3fn, for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation follows the pages' statement of the problem:
 *   - ONNX Runtime PR #29912 (PagedAttention), "Summary of Changes": query,
 *     key_cache / value_cache typed float16 | int8 | float8e4m3fn, the block
 *     table and block size, head_sink, k_scale / v_scale with
 *     k_quant_type / v_quant_type NONE | PER_TENSOR | PER_CHANNEL, the
 *     SEPARATE | LATENT cache layout with v_head_size, and graph safety
 *     (launch geometry and workspace from static shapes and the
 *     block_table.shape[1] * block_size capacity; per-step lengths read on
 *     the device);
 *   - ONNX Runtime PR #33707 (INT8 DynamicSparseAttention), "Summary of
 *     Changes" sections 1-2: per-row selected candidate lists with invalid
 *     entries, a finite non-negative softmax scale, the split-K partial
 *     (running maximum in natural-log units, running sum, value-scaled
 *     accumulator) and its merge, a statically sized workspace;
 *   - ONNX Runtime PR #29912, "Summary of Changes", paged decode kernel:
 *     the logit soft cap and the sliding window (their arithmetic is not
 *     spelled out there; the definition below takes the usual forms);
 *   - onnx-genai PR #1350 "Summary": the split count comes from the static
 *     capacity and the row count so that about one occupancy wave of CTAs
 *     runs, never from live lengths.
 *
 * Definition.  For row r (one decode query token) and query head h with KV
 * head g = h / (num_heads / num_kv_heads):
 *   len    = clamp(seq_lens[r], 0, max_blocks_per_row * block_size)
 *   lo     = max(0, len - sliding_window) when sliding_window > 0, else 0
 *   T      = [lo, len) for dense rows (max_candidates == 0); for gathered rows
 *            the list candidates[r][0 : clamp(num_candidates[r], 0,
 *            max_candidates)] in list order, keeping entries in [lo, len)
 *            (duplicates count twice)
 *   slot t = block_table[r][t / block_size] * block_size + t % block_size
 *   x_t    = softmax_scale * sum_d Q[r,h,d] * K^[slot t, g, d], then with
 *            softcap c > 0:  x_t <- c * tanh(x_t / c)
 *   O      = sum_t exp(x_t - m) V^[slot t, g, :] / sum_t exp(x_t - m),
 *            m = max_t x_t;  lse = m + log sum_t exp(x_t - m)
 *   sink   O <- O / (1 + exp(head_sink[h] - lse)) when head_sink != NULL
 *   empty  T = {} gives O = 0 and lse = -inf.
 * K^ / V^ are the stored codes times their scale (x = code * scale; per
 * tensor: scale[0]; per channel: scale[g * dim + d]).  LATENT: one cache
 * [.., 1 row per token and KV head, head_size]; V^ is the first v_head_size
 * channels of the K row, with the K scales.
 *
 * Several query tokens per row (query_tokens = T > 1; the multi-token decode
 * of speculative and chunked steps, ONNX Runtime PR #33707 "Testing": 1, 3
 * and 8 query rows of one sequence).  A row is then one sequence with T new
 * query tokens that share its block-table row; seq_lens[r] counts all T of
 * them, and token j (0 <= j < T) attends causally:
 *   len_j  = max(0, len - (T - 1 - j)),  T_j = [lo_j, len_j),
 *   lo_j   = max(0, len_j - sliding_window) when sliding_window > 0, else 0
 * query is [num_rows, T, num_heads, head_size], out [num_rows, T, num_heads,
 * v_head_size], lse [num_rows, T, num_heads]; the result for token j is the
 * definition above with len_j (each token's window ends at its own
 * position).  Every KV tile a CTA reads serves all T tokens of its query
 * heads (the (token, head) pairs of a KV head fill the 16-wide MFMA tile:
 * T * group <= 16 reads each tile once).  Dense rows, the SEPARATE layout,
 * 1 <= T <= 16.
 *
 * Memory layouts (all row-major, device memory unless stated):
 *   query        [num_rows, num_heads, head_size]              float16
 *   key_cache    [num_pool_blocks, block_size, num_kv_heads, head_size]
 *   value_cache  [num_pool_blocks, block_size, num_kv_heads, v_head_size]
 *                (NULL for LATENT)                              cache_dtype
 *   block_table  [num_rows, max_blocks_per_row]                int32
 *   seq_lens     [num_rows]                                    int32
 *   candidates   [num_rows, max_candidates]                    int32
 *   num_candidates [num_rows]                                  int32
 *   k_scale      [1] (PER_TENSOR) or [num_kv_heads, head_size] (PER_CHANNEL)
 *   v_scale      [1] or [num_kv_heads, v_head_size]            float32
 *   head_sink    [num_heads]                                   float32
 *   out          [num_rows, num_heads, v_head_size]            out_dtype
 *   lse_out      [num_rows, num_heads]                         float32
 *   workspace    partial accumulators [num_rows, num_heads, S, v_head_size]
 *                float32 followed by (m, l) pairs [num_rows, num_heads, S, 2]
 *
 * Ownership and threading.  The caller allocates and frees every buffer; the
 * library never allocates, frees or synchronises.  Calls enqueue work on the
 * caller's HIP stream and return; buffers must stay valid until that work
 * completes.  Two calls that share a workspace must not overlap in time.
 * The only library state is a per-device cache of the CU count and kernel
 * occupancy (thread-safe).
 *
 * Errors.  Static arguments are checked before anything is enqueued; on any
 * error nothing was enqueued.  pkv_last_error() returns a message naming the
 * offending argument (thread-local).  Device-resident data cannot be checked
 * without a synchronisation, so it has defined semantics instead: seq_lens
 * are clamped to [0, capacity]; num_candidates to [0, max_candidates];
 * candidate indices outside [lo, len) are skipped; a block-table entry
 * outside [0, num_pool_blocks) makes its tokens contribute nothing (they are
 * never read); block-table entries past the live length are never read.
 *
 * Graph safety.  The launch configuration depends only on pkv_problem and
 * pkv_geometry, never on device data, and no call records a memset or a
 * host synchronisation, so a call may be captured in a hipGraph and replayed
 * with different seq_lens / candidates / block tables.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,          /* an argument is invalid (null, out of range, ...) */
  PKV_EUNSUPPORTED = 2,    /* valid, but no compiled kernel covers it */
  PKV_EALIGN = 3,          /* a pointer is not aligned as required */
  PKV_EWORKSPACE = 4,      /* workspace_bytes smaller than required */
  PKV_EHIP = 5             /* the HIP runtime reported an error */
} pkv_status;

typedef enum { PKV_F16 = 0, PKV_I8 = 1, PKV_FP8_E4M3FN = 2, PKV_F32 = 3 } pkv_dtype;
typedef enum { PKV_QUANT_NONE = 0, PKV_QUANT_PER_TENSOR = 1, PKV_QUANT_PER_CHANNEL = 2 } pkv_quant;
typedef enum { PKV_SEPARATE = 0, PKV_LATENT = 1 } pkv_layout;

/* Static description of one decode step; nothing here depends on live data.
 * Supported: (head_size, v_head_size) in {(64,64), (128,128), (256,256)} for
 * SEPARATE and (576,512) for LATENT; block_size a power of two >= 16;
 * cache_dtype F16 (any quant), I8 or FP8_E4M3FN (quant PER_TENSOR or
 * PER_CHANNEL); out_dtype F16 or F32; num_heads a multiple of num_kv_heads;
 * capacity max_blocks_per_row * block_size and max_candidates at most 2^30;
 * one row's query block, query_tokens * num_heads * head_size FP16 values,
 * under 2^30 bytes (PKV_EUNSUPPORTED otherwise). */
typedef struct {
  int32_t num_rows;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t v_head_size;
  int32_t block_size;
  int32_t max_blocks_per_row;
  int32_t num_pool_blocks;
  int32_t max_candidates;  /* 0: dense rows [0, seq_len); > 0: gathered rows */
  int32_t cache_dtype;     /* pkv_dtype */
  int32_t out_dtype;       /* pkv_dtype: PKV_F16 or PKV_F32 */
  int32_t k_quant;         /* pkv_quant */
  int32_t v_quant;         /* pkv_quant; LATENT: ignored (V uses the K scales) */
  int32_t layout;          /* pkv_layout */
  int32_t sliding_window;  /* > 0: attend to the last sliding_window positions only; 0: all */
  float softcap;           /* > 0: logit soft cap c, x <- c tanh(x / c); 0: none */
  int32_t query_tokens;    /* query tokens per row T (0 or 1: one); T > 1: see below */
} pkv_problem;

/* Optional knobs of split_geometry (pass NULL for all defaults; 0 = default). */
typedef struct {
  int32_t num_cus;          /* compute units; 0 = query the current device */
  int32_t ctas_per_cu;      /* resident CTAs per CU; 0 = occupancy query */
  int32_t splits_override;  /* > 0: use this split count (clipped to the caps) */
  int32_t min_chunk;        /* smallest positions per split (multiple of 16) */
  int32_t max_splits;       /* cap on the split count */
  int32_t waves;            /* target = waves * num_cus * ctas_per_cu CTAs */
  int32_t balance;          /* 0: auto (live-balanced for 16..1024 rows), 1: live-
                               balanced (up to 1024 rows), 2: static; rows whose
                               positions could sum to 2^31 always use static */
  int32_t kv_heads_per_cta; /* 0: auto (4 when allowed, else 1); 1; 4 or 8: one CTA takes
                               that many neighbouring KV heads, one per wave (dense rows,
                               SEPARATE layout, num_kv_heads a multiple of it, at most 16
                               (token, head) slots per KV head; with 4, up to 32 slots at
                               head sizes up to 128, each wave taking both 16-slot blocks) */
} pkv_geometry_opts;

/* Launch geometry; produced by split_geometry, consumed unchanged. */
typedef struct {
  int32_t num_splits;       /* S: CTAs per (row, KV head, head block) */
  int32_t min_chunk;        /* positions per active split are >= this */
  int32_t threads;          /* threads per CTA of the split kernel */
  int32_t head_blocks;      /* ceil(query_tokens * group / 16): (token, head) slots go 16
                               per MFMA column tile */
  int32_t grid_x, grid_y, grid_z;  /* split-kernel grid (1-D: grid_y = grid_z = 1) */
  int32_t target_ctas;      /* active CTAs the live chunk size aims at (0: per-row rule) */
  int32_t kv_heads_per_cta; /* 1, 4 or 8 (the several-KV-head CTAs of split_geometry's opts) */
  uint64_t workspace_bytes; /* bytes of workspace the calls below need */
} pkv_geometry;

/*
 * split_geometry -- choose the split count S from static shapes only.
 *
 * units = num_rows * num_kv_heads * ceil(slots / 16) with one KV head per CTA,
 *         num_rows * (num_kv_heads / kv_heads_per_cta) with several (slots =
 *         query_tokens * group, the (token, head) slots of a KV head);
 *         kv_heads_per_cta is 4 when the problem allows it (dense rows, SEPARATE
 *         layout, a multiple of four KV heads, head size <= 128, slots <= 16 --
 *         or slots <= 32 with an FP16 cache or query_tokens > 1: the cache
 *         keeps the KV heads of a token side by side, and a CTA whose four
 *         waves read four neighbouring heads of the same records streams
 *         faster than four CTAs reading one head each) and opts do not ask
 *         for 1;
 * cap   = max_blocks_per_row * block_size (dense; with a sliding window W
 *         at most W + T - 1 + 15, the positions from the first token's
 *         window start rounded down to a multiple of 16) or max_candidates
 *         (gathered);
 *         resident = num_cus * ctas_per_cu.
 * Dense rows (onnx-genai PR #1350 "Summary"; target = waves * resident):
 *   S = min(ceil(target / units), ceil(cap / min_chunk), max_splits)
 *   (see below for the factor 4 of the live-balanced mode)
 * Gathered rows (ONNX Runtime PR #33707 section 2, split count rule): the
 *   unit of work is a 64-candidate tile; tiles-per-split is the smallest
 *   power of two for which ceil(tiles / tps) * units <= waves * resident;
 *   S = min(ceil(tiles / tps), max_splits).
 * With the automatic split count and min_chunk, rows of at most 256
 * positions (cap <= 256) take S = 1: one launch with the direct output.
 * A positive splits_override replaces the automatic count (then clipped to
 * [1, max_splits] and to ceil(cap / 16)).
 * On the device (graph safe, from live data): with target_ctas > 0 every CTA
 * sums the live positions of all rows (npos_r = clamped seq_len, or clamped
 * num_candidates for gathered rows) and takes one chunk
 *   c = max(min_chunk, round_up_16(ceil(sum_r npos_r * units_per_row / target_ctas)))
 * so that about target_ctas CTAs of similar work run; row r then uses
 * n_r = clamp(ceil(npos_r / c), 1, S) splits, and the 1-D grid's CTAs take
 * the work items (row, KV head x head block, split) in that order (the
 * grid holds min(units * S, target_ctas + units) CTAs; spare ones exit).
 * A row's n_r splits share its positions evenly in 16-position steps;
 * splits beyond n_r publish an empty partial.
 * Static mode (target_ctas = 0: opts.balance = 2, fewer than 16 rows under
 * auto, or more than 1024 rows): CTA i is item i of the (row, unit,
 * split < S) list and split k covers positions [k c, (k + 1) c) with
 * c = max(min_chunk, round_up_16(ceil(cap / S))); splits past the live length publish an
 * empty partial.  In the live-balanced
 * mode the automatic S allows rows up to four times the mean work:
 *   S = min(ceil(4 * target / units), ceil(cap / min_chunk), max_splits).
 * Defaults: max_splits 64.  min_chunk: 64, raised to the smallest power of
 * two c for which a split's partial P = group * (v_head_size + 2) * 4 bytes
 * is at most an eighth of the KV bytes of c positions, if the grid then
 * still gives every CU a CTA (units * ceil(cap / c) >= num_cus; two CTAs,
 * >= 2 * num_cus, with several KV heads per CTA); else to
 * the smallest c with P at most a quarter of them, if the grid then still
 * holds a quarter of the resident CTAs (units * ceil(cap / c) * 4 >=
 * resident); else kept at 64 -- a latency-bound step gains from more,
 * shorter splits.  P and the KV bytes are those of a work unit (four KV
 * heads in the four-head mode).  waves: 2 in the live-balanced mode with
 * one KV head per CTA when 2 P is less than the KV bytes of min_chunk
 * positions, else 1.  In the several-KV-head mode with query_tokens > 1 or
 * 17-32 slots per KV head: ctas_per_cu defaults to 1 (except for 17-32
 * slots over a one-byte cache), and in the live-balanced mode target =
 * resident - units when units <= resident / 2 (so that the rounded per-row
 * split counts fit one round); with 17-32 slots min_chunk follows the
 * quarter rule alone, on the KV bytes the positions would take in FP16.
 * Returns PKV_EINVAL / PKV_EUNSUPPORTED as paged_decode_attention would, or
 * PKV_EHIP if the device query fails.  Does not touch device memory.
 */
pkv_status split_geometry(const pkv_problem* problem, const pkv_geometry_opts* opts,
                          pkv_geometry* out);

/*
 * paged_decode_attention -- one decode step: the split kernel writes per-split
 * partials into `workspace`, then the combine kernel merges them (fixed split
 * order, so results are bitwise repeatable), applies the head sink and writes
 * `out` (and `lse_out` if not NULL).  Two kernel launches on `stream`
 * (a hipStream_t; NULL = the default stream); no allocation, no memset, no
 * synchronisation.  With one split (geometry->num_splits == 1, e.g. many
 * rows) the split kernel writes `out` and `lse_out` itself, bitwise what
 * the combine would write, in one launch; the workspace is then unused.
 *
 * Numerics (ONNX Runtime PR #33707, "Numerics" and its review thread): the
 * key scale is folded into an FP16 query and the probabilities enter the PV
 * products as FP16 high + residual tiles (scaled by 16).  Each CTA bounds
 * the logit error of the folding per head and recomputes its partial on an
 * FP32 path (unfolded query, exact running maximum, FP32 sums) when the
 * bound exceeds 0.125 nats, or when quantised values with
 * max|v_scale| * max|code| * positions >= 2^17 meet a probability below the
 * FP16 tile's normal range.  Accuracy against an FP64 reference on
 * unit-variance values: max abs error <= 2e-3, mean <= 2e-4.
 *
 * Alignment: query, key_cache, value_cache, out, workspace and per-channel
 * scale arrays 16-byte aligned; integer arrays, per-tensor scales,
 * head_sink and lse_out 4-byte aligned.  softmax_scale must be finite and
 * >= 0.  workspace_bytes >= geometry->workspace_bytes.  The geometry must be
 * the one split_geometry returned for this problem.
 */
pkv_status paged_decode_attention(const pkv_problem* problem, const pkv_geometry* geometry,
                                  const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* candidates,
                                  const int32_t* num_candidates, const float* k_scale,
                                  const float* v_scale, float softmax_scale,
                                  const float* head_sink, void* out, float* lse_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_partials -- the split kernel alone: writes the per-split
 * partials (value-scaled accumulator, running maximum in natural-log units,
 * running sum) into `workspace` and nothing else.  split_combine then turns
 * them into the output.  Partials of disjoint position ranges (for example
 * computed on different devices for one long row) merge exactly the same
 * way.  Same arguments and rules as paged_decode_attention.
 */
pkv_status paged_decode_partials(const pkv_problem* problem, const pkv_geometry* geometry,
                                 const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* candidates,
                                 const int32_t* num_candidates, const float* k_scale,
                                 const float* v_scale, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * split_combine -- merge the S partials of every (row, query head) in split
 * order: M = max_k m_k, w_k = exp(m_k - M), L = sum_k w_k l_k,
 * O = sum_k w_k acc_k / L, lse = M + log L (empty: O = 0, lse = -inf), then
 * the exact head-sink rescale O <- O / (1 + exp(head_sink[h] - lse))
 * (ONNX Runtime PR #29912, ApplyHeadSink).  One launch on `stream`.
 */
pkv_status split_combine(const pkv_problem* problem, const pkv_geometry* geometry,
                         const void* workspace, size_t workspace_bytes, const float* head_sink,
                         void* out, float* lse_out, void* stream);

/*
 * paged_decode_attention_noalloc -- paged_decode_attention for callers that
 * cannot allocate device memory (code under hipGraph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same operation, arguments and
 * kernels, without the workspace argument.  The partials live in a device
 * array of PKV_NOALLOC_WORKSPACE_BYTES (64 MiB) that the library holds on
 * every GPU it runs on until the process ends; the call allocates, frees
 * and memsets nothing.  The array's device address is resolved once per
 * device (hipGetSymbolAddress) with that device current.
 *
 * Limit: a geometry whose workspace_bytes exceed PKV_NOALLOC_WORKSPACE_BYTES
 * is rejected with PKV_EWORKSPACE before anything is enqueued (fewer rows or
 * a smaller splits_override fit; e.g. 16 rows x 32 heads x 64 splits x 128
 * channels need 17 MB).  The array keeps the last call's partials; no call
 * needs it cleared.  All calls on one GPU share its one array, so calls that
 * overlap in time on one GPU (two streams, or two host threads) race and
 * must be ordered by the caller.  Results are bitwise those of
 * paged_decode_attention with the same geometry.
 */
#define PKV_NOALLOC_WORKSPACE_BYTES (64u << 20)

pkv_status paged_decode_attention_noalloc(const pkv_problem* problem,
                                          const pkv_geometry* geometry, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const int32_t* candidates,
                                          const int32_t* num_candidates, const float* k_scale,
                                          const float* v_scale, float softmax_scale,
                                          const float* head_sink, void* out, float* lse_out,
                                          void* stream);

/*
 * reshape_and_cache -- quantise-on-write of new K/V rows into the paged cache
 * (ONNX Runtime PR #29912, "Summary of Changes": ReshapeAndCache writes each
 * new token at the slot its slot_mapping entry names, quantised with
 * k_scale / v_scale at the granularity k_quant / v_quant give).
 *
 * For token t with slot = slot_mapping[t] in [0, num_pool_blocks *
 * block_size), KV head g and channel d:
 *   v    = float32(x[t, g, d]) / scale[g, d]   (FP32, correctly rounded;
 *          scale = 1 for PKV_QUANT_NONE, scale[0] per tensor)
 *   code = INT8: clamp(round-half-even(v), -128, 127)
 *          FP8 e4m3fn: the nearest finite value, ties to the even code,
 *            saturating at +-448, the sign kept on a rounding to zero
 *          FP16: v rounded to half (round-half-even)
 *   key_cache[slot / block_size][slot % block_size][g][d] = code (and the
 *   same for value / value_cache).  A token whose slot lies outside the
 *   pool is skipped (nothing is written for it).  LATENT: one cache; `value`
 *   and `value_cache` must be NULL and the row is quantised with k_scale.
 *
 * Layouts (row-major, device memory):
 *   key          [num_tokens, num_kv_heads, head_size]     float16
 *   value        [num_tokens, num_kv_heads, v_head_size]   float16
 *   slot_mapping [num_tokens]                              int64
 *   caches and scales as for paged_decode_attention.
 * Only the problem's num_kv_heads, head_size, v_head_size, block_size,
 * num_pool_blocks, cache_dtype, k_quant, v_quant and layout are used.
 * Alignment: key, value and the caches 16-byte aligned, head_size and
 * v_head_size multiples of 8 (as everywhere), per-channel scales 16-byte
 * and per-tensor scales 4-byte aligned, slot_mapping 8-byte aligned.
 * Two tokens mapped to one slot race (the result is one of them).  One
 * launch on `stream` (none when num_tokens == 0); no allocation, memset or
 * synchronisation; graph safe.  Errors as for paged_decode_attention.
 */
pkv_status reshape_and_cache(const pkv_problem* problem, int32_t num_tokens, const void* key,
                             const void* value, const int64_t* slot_mapping,
                             const float* k_scale, const float* v_scale, void* key_cache,
                             void* value_cache, void* stream);

/* Static string for a status code. */
const char* pkv_status_string(pkv_status status);

/* Message describing the most recent failure on the calling thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
