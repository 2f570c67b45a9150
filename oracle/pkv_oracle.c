/*
 * pkv_oracle.c -- plain FP64 CPU reference for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library never
 * links, includes or calls it, and this file includes nothing of the GPU
 * library: the two share no code, headers, tables or constants.
 *
 * What it computes (one query token per row, grouped-query heads):
 *
 *   For row r and query head h with KV head g = h / (heads / kv_heads):
 *     len  = clamp(seq_lens[r], 0, max_blocks_per_row * block_size)
 *     lo   = max(0, len - W) with a sliding window of W > 0 tokens, else 0
 *     T    = [lo, len)                                  (dense rows), or
 *            candidates[r][0 : num_candidates[r]] in list order, keeping only
 *            entries in [lo, len)                         (gathered rows)
 *     slot(t) = block_table[r][t / block_size] * block_size + t % block_size
 *     x_t  = softmax_scale * sum_d Q[r,h,d] * Khat[slot(t), g, d]
 *            then, with a soft cap c > 0:  x_t <- c * tanh(x_t / c)
 *     m    = max_t x_t ;  w_t = exp(x_t - m) ;  l = sum_t w_t ;  lse = m + log l
 *     O[c] = sum_t w_t * Vhat[slot(t), g, c] / l
 *     with a head sink s_h:  O <- O / (1 + exp(s_h - lse))
 *     empty T: O = 0, lse = -inf.
 *
 *   Khat / Vhat are the stored codes decoded exactly and multiplied by the
 *   scale (per tensor: one float; per channel: one float per [kv_head, d]).
 *   In the latent layout there is one cache; V is the first v_head_size
 *   channels of the same row that supplies K, with K's scales.
 *
 * Sources (the pages, by section):
 *   - ONNX Runtime PR #33707 (DynamicSparseAttention INT8 KV cache),
 *     "Summary of Changes" section 1 (key scale folded into the query, value
 *     scale applied after accumulation, natural-log softmax) and its test
 *     description: an FP64 reference evaluated on exactly the inputs the
 *     kernel gets, with weights taken relative to the maximum score;
 *     section 2 (split-K partials of
 *     running maximum, running sum and accumulator, merged afterwards;
 *     selected candidate lists with invalid entries).
 *   - ONNX Runtime PR #29912 (PagedAttention), "Summary of Changes": the
 *     block table and block size, k_scale / v_scale with PER_TENSOR or
 *     PER_CHANNEL granularity, the float8e4m3fn cache type, the LATENT layout
 *     (V = leading v_head_size channels of the row that supplies K), and the
 *     exact post-hoc head-sink rescale 1 / (1 + exp(s_h - lse)); its paged
 *     decode kernel also supports a logit soft cap and a sliding window, whose
 *     arithmetic the page does not spell out (readings below).
 *   - The split-and-merge variant (oracle_paged_decode with chunk > 0) follows
 *     the flash-decoding partial/merge description of PR #33707 section 2 and
 *     onnx-genai PR #1350 "Summary"; it exists to pin the invariant that
 *     splitting does not change the result.
 *
 * Readings where the pages are silent (listed in the design notes):
 *   cache layout [num_blocks, block_size, kv_heads, head_size]; per-channel
 *   scales of shape [kv_heads, head_size]; symmetric dequantisation
 *   x = code * scale; OCP e4m3fn decoding (bias 7, no infinities, S.1111.111
 *   is NaN); head_sink per query head, in scaled-logit units; seq_len clamped
 *   to the block-table capacity; duplicate candidates count twice; the soft
 *   cap acts on the scaled logit, x <- c tanh(x / c); a window of W tokens
 *   keeps the W most recent positions [len - W, len) of the row (the decode
 *   query is the token at position len - 1).
 *
 * Numerics: every decoded input is exact in double; sums run in logical token
 * order with plain loops, so permuting the physical blocks cannot change a
 * single bit of the result.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_I8 = 1, OR_FP8E4M3 = 2 };
enum { OR_QNONE = 0, OR_QTENSOR = 1, OR_QCHANNEL = 2 };

/* IEEE binary16 bit pattern -> double (exact). */
double oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1f;
  int m = bits & 0x3ff;
  double v;
  if (e == 0x1f) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -24);             /* subnormal: m * 2^-24 */
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* OCP float8 e4m3fn bit pattern -> double (exact).  NaN for S.1111.111. */
double oracle_fp8e4m3_to_f64(uint8_t bits) {
  int sign = (bits >> 7) & 1;
  int e = (bits >> 3) & 0xf;
  int m = bits & 0x7;
  double v;
  if (e == 0xf && m == 0x7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -9);              /* 2^-6 * m/8 */
  } else {
    v = ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7) */
  }
  return sign ? -v : v;
}

/* One stored code, decoded exactly (no scale). */
double oracle_decode_code(int dtype, uint32_t code) {
  switch (dtype) {
    case OR_F16: return oracle_f16_to_f64((uint16_t)code);
    case OR_I8: return (double)(int8_t)(uint8_t)code;
    case OR_FP8E4M3: return oracle_fp8e4m3_to_f64((uint8_t)code);
    default: return NAN;
  }
}

/* Dequantised value: code * scale, exact in double. */
double oracle_dequant(int dtype, uint32_t code, float scale) {
  return oracle_decode_code(dtype, code) * (double)scale;
}

typedef struct {
  /* shapes */
  int rows, heads, kv_heads, head_size, v_head_size;
  int block_size, max_blocks_per_row, num_pool_blocks, max_candidates;
  int cache_dtype, k_quant, v_quant, latent;
  /* inputs */
  const uint16_t* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* candidates;
  const int32_t* num_candidates;
  const float* k_scale;
  const float* v_scale;
  double softmax_scale;
  double softcap;
  int window;
  const float* head_sink;
  int chunk;
  /* outputs */
  double* out;
  double* lse;
  /* work list */
  const int32_t* unit_list; /* (row, kv_head) pairs flattened as row*kv_heads+g */
  int n_units;
  int next_unit;
  int error;
  pthread_mutex_t lock;
} oracle_job;

static uint32_t load_code(const void* base, int dtype, size_t index) {
  if (dtype == OR_F16) return ((const uint16_t*)base)[index];
  return ((const uint8_t*)base)[index];
}

static double scale_of(int quant, const float* scale, int g, int dim, int d) {
  if (quant == OR_QNONE) return 1.0;
  if (quant == OR_QTENSOR) return (double)scale[0];
  return (double)scale[(size_t)g * dim + d];
}

/* Dequantised K element of token slot `slot`, KV head g, channel d. */
static double khat(const oracle_job* J, int64_t slot, int g, int d) {
  size_t idx = ((size_t)slot * J->kv_heads + g) * J->head_size + d;
  return oracle_decode_code(J->cache_dtype, load_code(J->key_cache, J->cache_dtype, idx)) *
         scale_of(J->k_quant, J->k_scale, g, J->head_size, d);
}

/* Dequantised V element.  Latent layout: the first v_head_size channels of the
 * K row, with the K scales. */
static double vhat(const oracle_job* J, int64_t slot, int g, int c) {
  if (J->latent) return khat(J, slot, g, c);
  size_t idx = ((size_t)slot * J->kv_heads + g) * J->v_head_size + c;
  return oracle_decode_code(J->cache_dtype, load_code(J->value_cache, J->cache_dtype, idx)) *
         scale_of(J->v_quant, J->v_scale, g, J->v_head_size, c);
}

/* Logical token list T for row r.  Returns its length; -1 on a block id out of
 * range (the inputs are invalid). */
static int token_list(const oracle_job* J, int r, int32_t* T, int64_t* slots) {
  int64_t cap = (int64_t)J->max_blocks_per_row * J->block_size;
  int64_t len = J->seq_lens[r];
  if (len < 0) len = 0;
  if (len > cap) len = cap;
  int64_t lo = 0;
  if (J->window > 0 && len > J->window) lo = len - J->window;
  int n = 0;
  if (J->max_candidates == 0) {
    for (int64_t t = lo; t < len; ++t) T[n++] = (int32_t)t;
  } else {
    int nc = J->num_candidates[r];
    if (nc < 0) nc = 0;
    if (nc > J->max_candidates) nc = J->max_candidates;
    for (int j = 0; j < nc; ++j) {
      int32_t c = J->candidates[(size_t)r * J->max_candidates + j];
      if (c >= lo && c < len) T[n++] = c;
    }
  }
  for (int i = 0; i < n; ++i) {
    int32_t t = T[i];
    int32_t blk = J->block_table[(size_t)r * J->max_blocks_per_row + t / J->block_size];
    if (blk < 0 || blk >= J->num_pool_blocks) return -1;
    slots[i] = (int64_t)blk * J->block_size + t % J->block_size;
  }
  return n;
}

/* One (row, kv head) unit: every query head of the group. */
static int run_unit(oracle_job* J, int r, int g, int32_t* T, int64_t* slots, double* x,
                    double* acc) {
  const int group = J->heads / J->kv_heads;
  const int D = J->head_size, VD = J->v_head_size;
  int n = token_list(J, r, T, slots);
  if (n < 0) return -1;
  for (int hh = 0; hh < group; ++hh) {
    const int h = g * group + hh;
    double* o = J->out + ((size_t)r * J->heads + h) * VD;
    double* lse = J->lse + (size_t)r * J->heads + h;
    const uint16_t* q = J->query + ((size_t)r * J->heads + h) * D;
    if (n == 0) {
      for (int c = 0; c < VD; ++c) o[c] = 0.0;
      *lse = -INFINITY;
      continue;
    }
    /* scores */
    for (int i = 0; i < n; ++i) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += oracle_f16_to_f64(q[d]) * khat(J, slots[i], g, d);
      x[i] = J->softmax_scale * dot;
      if (J->softcap > 0.0) x[i] = J->softcap * tanh(x[i] / J->softcap);
    }
    double M, L;
    for (int c = 0; c < VD; ++c) o[c] = 0.0;
    if (J->chunk <= 0) {
      /* monolithic: max-subtracted weights over the whole list */
      M = -INFINITY;
      for (int i = 0; i < n; ++i) M = x[i] > M ? x[i] : M;
      L = 0.0;
      for (int i = 0; i < n; ++i) {
        double w = exp(x[i] - M);
        L += w;
        for (int c = 0; c < VD; ++c) o[c] += w * vhat(J, slots[i], g, c);
      }
      for (int c = 0; c < VD; ++c) o[c] /= L;
    } else {
      /* split variant: partial (m_k, l_k, acc_k) per consecutive chunk of the
       * list, then the merge M = max m_k, w_k = exp(m_k - M),
       * L = sum w_k l_k, O = sum w_k acc_k / L. */
      int nchunks = (n + J->chunk - 1) / J->chunk;
      M = -INFINITY;
      for (int k = 0; k < nchunks; ++k) {
        int b = k * J->chunk, e = b + J->chunk < n ? b + J->chunk : n;
        double mk = -INFINITY;
        for (int i = b; i < e; ++i) mk = x[i] > mk ? x[i] : mk;
        M = mk > M ? mk : M;
      }
      L = 0.0;
      for (int k = 0; k < nchunks; ++k) {
        int b = k * J->chunk, e = b + J->chunk < n ? b + J->chunk : n;
        double mk = -INFINITY;
        for (int i = b; i < e; ++i) mk = x[i] > mk ? x[i] : mk;
        double lk = 0.0;
        for (int c = 0; c < VD; ++c) acc[c] = 0.0;
        for (int i = b; i < e; ++i) {
          double w = exp(x[i] - mk);
          lk += w;
          for (int c = 0; c < VD; ++c) acc[c] += w * vhat(J, slots[i], g, c);
        }
        double wk = exp(mk - M);
        L += wk * lk;
        for (int c = 0; c < VD; ++c) o[c] += wk * acc[c];
      }
      for (int c = 0; c < VD; ++c) o[c] /= L;
    }
    *lse = M + log(L);
    if (J->head_sink) {
      double f = 1.0 / (1.0 + exp((double)J->head_sink[h] - *lse));
      for (int c = 0; c < VD; ++c) o[c] *= f;
    }
  }
  return 0;
}

static void* worker(void* arg) {
  oracle_job* J = (oracle_job*)arg;
  int64_t cap = (int64_t)J->max_blocks_per_row * J->block_size;
  int64_t nmax = J->max_candidates > 0 ? J->max_candidates : cap;
  int32_t* T = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nmax > 0 ? nmax : 1));
  int64_t* slots = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nmax > 0 ? nmax : 1));
  double* x = (double*)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)J->v_head_size);
  if (!T || !slots || !x || !acc) {
    pthread_mutex_lock(&J->lock);
    J->error = -2;
    pthread_mutex_unlock(&J->lock);
  } else {
    for (;;) {
      pthread_mutex_lock(&J->lock);
      int u = J->next_unit++;
      pthread_mutex_unlock(&J->lock);
      if (u >= J->n_units) break;
      int unit = J->unit_list[u];
      int rc = run_unit(J, unit / J->kv_heads, unit % J->kv_heads, T, slots, x, acc);
      if (rc) {
        pthread_mutex_lock(&J->lock);
        J->error = rc;
        pthread_mutex_unlock(&J->lock);
      }
    }
  }
  free(T);
  free(slots);
  free(x);
  free(acc);
  return NULL;
}

/*
 * Paged decode attention in FP64.
 *   query        [rows, heads, head_size] binary16 bit patterns
 *   key_cache    [num_pool_blocks, block_size, kv_heads, head_size] codes
 *   value_cache  [num_pool_blocks, block_size, kv_heads, v_head_size] codes,
 *                ignored for the latent layout
 *   block_table  [rows, max_blocks_per_row]
 *   seq_lens     [rows]
 *   candidates   [rows, max_candidates] (max_candidates > 0), else unused
 *   k_scale      [1] or [kv_heads, head_size]; v_scale [1] or
 *                [kv_heads, v_head_size]; unused for quant NONE
 *   head_sink    [heads] or NULL
 *   softcap      > 0: logit soft cap c; 0: none
 *   window       > 0: sliding window of that many tokens; 0: none
 *   chunk        0: monolithic softmax; > 0: split into chunks of `chunk`
 *                list entries, partials merged in FP64
 *   row_subset   optional list of rows to evaluate (others untouched)
 *   out          [rows, heads, v_head_size];  lse [rows, heads]
 * Returns 0, -1 for a block id outside the pool, -2 on allocation failure,
 * -3 for invalid shapes.
 */
int oracle_paged_decode(int rows, int heads, int kv_heads, int head_size, int v_head_size,
                        int block_size, int max_blocks_per_row, int num_pool_blocks,
                        int max_candidates, int cache_dtype, int k_quant, int v_quant,
                        int latent, const uint16_t* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_table,
                        const int32_t* seq_lens, const int32_t* candidates,
                        const int32_t* num_candidates, const float* k_scale,
                        const float* v_scale, double softmax_scale, const float* head_sink,
                        double softcap, int window, int chunk, int num_threads, const int32_t* row_subset,
                        int n_row_subset, double* out, double* lse) {
  if (rows < 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0 || head_size <= 0 ||
      v_head_size <= 0 || block_size <= 0 || max_blocks_per_row < 0 || max_candidates < 0)
    return -3;
  if (latent && v_head_size > head_size) return -3;
  if (cache_dtype < OR_F16 || cache_dtype > OR_FP8E4M3) return -3;
  if (!(softcap >= 0.0) || window < 0) return -3;
  oracle_job J;
  memset(&J, 0, sizeof(J));
  J.rows = rows; J.heads = heads; J.kv_heads = kv_heads; J.head_size = head_size;
  J.v_head_size = v_head_size; J.block_size = block_size;
  J.max_blocks_per_row = max_blocks_per_row; J.num_pool_blocks = num_pool_blocks;
  J.max_candidates = max_candidates; J.cache_dtype = cache_dtype; J.k_quant = k_quant;
  J.v_quant = latent ? k_quant : v_quant; J.latent = latent;
  J.query = query; J.key_cache = key_cache; J.value_cache = value_cache;
  J.block_table = block_table; J.seq_lens = seq_lens; J.candidates = candidates;
  J.num_candidates = num_candidates; J.k_scale = k_scale;
  J.v_scale = latent ? k_scale : v_scale; J.softmax_scale = softmax_scale;
  J.head_sink = head_sink; J.softcap = softcap; J.window = window; J.chunk = chunk; J.out = out; J.lse = lse;

  int nrows_eval = row_subset ? n_row_subset : rows;
  int32_t* units = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows_eval * kv_heads + 1));
  if (!units) return -2;
  int nu = 0;
  for (int i = 0; i < nrows_eval; ++i) {
    int r = row_subset ? row_subset[i] : i;
    if (r < 0 || r >= rows) { free(units); return -3; }
    for (int g = 0; g < kv_heads; ++g) units[nu++] = r * kv_heads + g;
  }
  J.unit_list = units;
  J.n_units = nu;
  pthread_mutex_init(&J.lock, NULL);
  if (num_threads < 1) num_threads = 1;
  if (num_threads > nu) num_threads = nu > 0 ? nu : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)num_threads);
  if (!th) { free(units); return -2; }
  int started = 0;
  for (int i = 1; i < num_threads; ++i)
    if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
  worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.lock);
  free(th);
  free(units);
  return J.error;
}
