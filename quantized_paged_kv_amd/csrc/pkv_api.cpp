// pkv_api.cpp -- the C ABI of libpkv: argument validation, split geometry
// and kernel dispatch.  See include/pkv.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

using pkv::kMaxBalancedRows;
// Fewer rows than this: the static decomposition (its first block reads do
// not wait for the live lengths, which matters more than balance there).
constexpr int kMinBalancedRows = 16;
// Rows of at most this many positions take one split (see split_geometry).
constexpr int64_t kOneSplitCap = 256;

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Query tokens per row and head slots per KV head ((token, head) pairs).
int qtok_of(const pkv_problem& p) { return p.query_tokens > 1 ? p.query_tokens : 1; }
int vgroup_of(const pkv_problem& p) { return qtok_of(p) * (p.num_heads / p.num_kv_heads); }

pkv::Variant variant_of(const pkv_problem& p) {
  pkv::Variant v;
  v.cache_dtype = p.cache_dtype;
  v.head_size = p.head_size;
  v.v_head_size = p.v_head_size;
  v.latent = p.layout == PKV_LATENT;
  v.gathered = p.max_candidates > 0;
  v.ext = p.sliding_window > 0 || p.softcap > 0.0f;
  v.kvp = 0;
  v.mt = qtok_of(p) > 1;
  v.vb = 1;
  return v;
}

// Several KV heads per CTA (split_kvp_kernel, kpc = 4 or 8): dense rows,
// separate caches, a multiple of kpc KV heads and at most 16 head slots
// (query heads x query tokens) per KV head -- or 32 (two head blocks per
// wave) with four KV heads per CTA and head sizes up to 128.
bool kvp_allowed(const pkv_problem& p, int kpc) {
  const int vg = vgroup_of(p);
  return (kpc == pkv::kKvHeadsPerCta || kpc == pkv::kKvHeadsPerCtaWide) &&
         p.layout == PKV_SEPARATE && p.max_candidates == 0 && p.num_kv_heads % kpc == 0 &&
         (vg <= 16 || (vg <= 32 && kpc == pkv::kKvHeadsPerCta && p.head_size <= 128));
}

// The kernel variant of a problem run with kv_per_cta KV heads per CTA.
pkv::Variant variant_for(const pkv_problem& p, int kv_per_cta) {
  pkv::Variant v = variant_of(p);
  v.kvp = kv_per_cta > 1 ? kv_per_cta : 0;
  v.vb = v.kvp ? ceil_div(vgroup_of(p), 16) : 1;
  return v;
}

// Work units per row: (KV head, 16-slot head block), or groups of kpc KV
// heads with all their head slots in the several-heads mode.
int64_t units_row_of(const pkv_problem& p, int kv_per_cta) {
  if (kv_per_cta > 1) return p.num_kv_heads / kv_per_cta;
  return (int64_t)p.num_kv_heads * ceil_div(vgroup_of(p), 16);
}

// Most positions one row can have: the candidate-list capacity (gathered
// rows), else the block-table capacity -- with a sliding window of W
// tokens at most W + T - 1 + 15 (T query tokens per row: the first token's
// window start to the last token), since a row's range starts at the window
// start rounded down to a multiple of 16 (so tiles never straddle a block).
int64_t positions_cap(const pkv_problem& p) {
  if (p.max_candidates > 0) return p.max_candidates;
  const int64_t cap = (int64_t)p.max_blocks_per_row * p.block_size;
  return p.sliding_window > 0
             ? std::min<int64_t>(cap, (int64_t)p.sliding_window + (qtok_of(p) - 1) + 15)
             : cap;
}

// Static checks of the problem description.
pkv_status check_problem(const pkv_problem* p) {
  if (!p) return fail(PKV_EINVAL, "problem is NULL");
  if (p->num_rows < 0) return fail(PKV_EINVAL, "num_rows < 0");
  if (p->num_heads <= 0 || p->num_kv_heads <= 0)
    return fail(PKV_EINVAL, "num_heads and num_kv_heads must be positive");
  if (p->num_heads % p->num_kv_heads)
    return fail(PKV_EINVAL, "num_heads (%d) is not a multiple of num_kv_heads (%d)", p->num_heads,
                p->num_kv_heads);
  if (p->head_size <= 0 || p->v_head_size <= 0) return fail(PKV_EINVAL, "head sizes must be positive");
  if (p->block_size < 16 || (p->block_size & (p->block_size - 1)))
    return fail(PKV_EUNSUPPORTED, "block_size (%d) must be a power of two >= 16", p->block_size);
  if (p->max_blocks_per_row <= 0) return fail(PKV_EINVAL, "max_blocks_per_row must be positive");
  if (p->num_pool_blocks <= 0) return fail(PKV_EINVAL, "num_pool_blocks must be positive");
  // positions are 32-bit on the device; at most 2^30 keeps every sum of two
  // of them in range
  if ((int64_t)p->max_blocks_per_row * p->block_size > (int64_t)1 << 30)
    return fail(PKV_EINVAL, "capacity max_blocks_per_row * block_size exceeds 2^30 positions");
  if (p->max_candidates > (1 << 30)) return fail(PKV_EINVAL, "max_candidates exceeds 2^30");
  if (p->max_candidates < 0) return fail(PKV_EINVAL, "max_candidates < 0");
  if (p->cache_dtype != PKV_F16 && p->cache_dtype != PKV_I8 && p->cache_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_EINVAL, "cache_dtype must be PKV_F16, PKV_I8 or PKV_FP8_E4M3FN");
  if (p->out_dtype != PKV_F16 && p->out_dtype != PKV_F32)
    return fail(PKV_EINVAL, "out_dtype must be PKV_F16 or PKV_F32");
  if (p->layout != PKV_SEPARATE && p->layout != PKV_LATENT)
    return fail(PKV_EINVAL, "layout must be PKV_SEPARATE or PKV_LATENT");
  for (int q : {p->k_quant, p->v_quant})
    if (q < PKV_QUANT_NONE || q > PKV_QUANT_PER_CHANNEL)
      return fail(PKV_EINVAL, "quant must be NONE, PER_TENSOR or PER_CHANNEL");
  if (p->cache_dtype != PKV_F16) {
    if (p->k_quant == PKV_QUANT_NONE)
      return fail(PKV_EINVAL, "a quantised cache needs k_quant PER_TENSOR or PER_CHANNEL");
    if (p->layout == PKV_SEPARATE && p->v_quant == PKV_QUANT_NONE)
      return fail(PKV_EINVAL, "a quantised cache needs v_quant PER_TENSOR or PER_CHANNEL");
  }
  if (p->query_tokens < 0) return fail(PKV_EINVAL, "query_tokens < 0");
  if (p->query_tokens > 1) {
    if (p->query_tokens > 16)
      return fail(PKV_EUNSUPPORTED, "query_tokens %d exceeds 16", p->query_tokens);
    if (p->max_candidates > 0 || p->layout != PKV_SEPARATE)
      return fail(PKV_EUNSUPPORTED,
                  "several query tokens per row need dense rows and the SEPARATE layout");
  }
  if ((int64_t)p->num_rows * qtok_of(*p) * p->num_heads > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "num_rows * query_tokens * num_heads is too large");
  // one row's query block is addressed through a buffer descriptor whose
  // range must stay below the past-the-range offset the kernels use
  if ((int64_t)qtok_of(*p) * p->num_heads * p->head_size * 2 >= (int64_t)1 << 30)
    return fail(PKV_EUNSUPPORTED, "query_tokens * num_heads * head_size * 2 bytes reach 2^30");
  if ((int64_t)p->num_rows * p->num_kv_heads * ceil_div(vgroup_of(*p), 16) * 64 >
      INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "num_rows * num_kv_heads * ceil(group / 16) is too large");
  if (p->sliding_window < 0) return fail(PKV_EINVAL, "sliding_window < 0");
  if (!(p->softcap >= 0.0f) || !std::isfinite(p->softcap))
    return fail(PKV_EINVAL, "softcap must be finite and >= 0");
  if (p->layout == PKV_LATENT && p->v_head_size > p->head_size)
    return fail(PKV_EINVAL, "LATENT needs v_head_size <= head_size");
  if (!pkv::variant_supported(variant_of(*p)))
    return fail(PKV_EUNSUPPORTED,
                "no kernel for head_size %d / v_head_size %d with layout %d (compiled: "
                "64/64, 128/128, 256/256 SEPARATE; 576/512 LATENT)",
                p->head_size, p->v_head_size, p->layout);
  return PKV_OK;
}

// The live-balanced decomposition: up to kMaxBalancedRows rows whose
// positions cannot sum to 2^31.
bool balance_fits(const pkv_problem& p) {
  return p.num_rows <= kMaxBalancedRows && (int64_t)p.num_rows * positions_cap(p) <= INT32_MAX;
}

uint64_t workspace_bytes_for(const pkv_problem& p, int S) {
  const uint64_t pairs = (uint64_t)p.num_rows * qtok_of(p) * p.num_heads;
  return pairs * S * p.v_head_size * sizeof(float) + pairs * S * 2 * sizeof(float);
}

// CTAs of the split kernel's 1-D grid.  Static mode: one per (row, unit,
// split).  Live-balanced mode: the work items are at most
// target + rows * units (each row rounds its split count up by less than one
// chunk), and never more than the static count.
int64_t grid_ctas_for(const pkv_problem& p, int S, int target, int kv_per_cta) {
  const int64_t units = (int64_t)p.num_rows * units_row_of(p, kv_per_cta);
  const int64_t all = units * S;
  return target > 0 ? std::min<int64_t>(all, (int64_t)target + units) : all;
}

// Per-device cache of (CU count, occupancy per variant).
struct DeviceInfo {
  int cus = 0;
  std::unordered_map<uint64_t, int> occupancy;
};
std::mutex g_dev_mu;
std::unordered_map<int, DeviceInfo> g_dev;

uint64_t variant_key(const pkv::Variant& v) {
  return ((uint64_t)v.cache_dtype << 48) | ((uint64_t)v.head_size << 32) |
         ((uint64_t)v.v_head_size << 16) | ((uint64_t)v.mt << 10) | ((uint64_t)v.vb << 8) |
         (v.kvp << 3) | (v.ext << 2) | (v.latent << 1) | v.gathered;
}

pkv_status device_numbers(const pkv::Variant& v, int* cus, int* occ) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& info = g_dev[dev];
  if (info.cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(PKV_EHIP, "cannot query the CU count of device %d", dev);
    info.cus = n;
  }
  *cus = info.cus;
  if (occ) {
    const uint64_t key = variant_key(v);
    auto it = info.occupancy.find(key);
    if (it == info.occupancy.end()) {
      int n = 0;
      if (pkv::split_occupancy(v, &n) != hipSuccess || n <= 0)
        return fail(PKV_EHIP, "occupancy query failed");
      it = info.occupancy.emplace(key, n).first;
    }
    *occ = it->second;
  }
  return PKV_OK;
}

pkv_status check_geometry(const pkv_problem& p, const pkv_geometry* g) {
  if (!g) return fail(PKV_EINVAL, "geometry is NULL");
  if (g->num_splits < 1 || g->num_splits > pkv::kMaxSplits)
    return fail(PKV_EINVAL, "geometry num_splits %d outside [1, %d]", g->num_splits, pkv::kMaxSplits);
  if (g->min_chunk < 16 || g->min_chunk % 16)
    return fail(PKV_EINVAL, "geometry min_chunk %d is not a positive multiple of 16", g->min_chunk);
  const pkv::Variant var = variant_for(p, g->kv_heads_per_cta);
  if (g->head_blocks != ceil_div(vgroup_of(p), 16) || g->threads != pkv::threads_of(var) ||
      (g->kv_heads_per_cta != 1 && !kvp_allowed(p, g->kv_heads_per_cta)) ||
      g->grid_x != grid_ctas_for(p, g->num_splits, g->target_ctas, g->kv_heads_per_cta) || g->grid_y != 1 ||
      g->grid_z != 1 || g->workspace_bytes != workspace_bytes_for(p, g->num_splits) ||
      g->target_ctas < 0 || (g->target_ctas > 0 && !balance_fits(p)))
    return fail(PKV_EINVAL, "geometry does not belong to this problem (call split_geometry)");
  return PKV_OK;
}

struct Ptrs {
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* candidates;
  const int32_t* num_candidates;
  const float* k_scale;
  const float* v_scale;
};

pkv_status check_inputs(const pkv_problem& p, const Ptrs& x, float softmax_scale) {
  if (!x.query) return fail(PKV_EINVAL, "query is NULL");
  if (!x.key_cache) return fail(PKV_EINVAL, "key_cache is NULL");
  if (p.layout == PKV_SEPARATE && !x.value_cache) return fail(PKV_EINVAL, "value_cache is NULL");
  if (p.layout == PKV_LATENT && x.value_cache)
    return fail(PKV_EINVAL, "value_cache must be NULL for the LATENT layout");
  if (!x.block_table) return fail(PKV_EINVAL, "block_table is NULL");
  if (!x.seq_lens) return fail(PKV_EINVAL, "seq_lens is NULL");
  if (p.max_candidates > 0 && (!x.candidates || !x.num_candidates))
    return fail(PKV_EINVAL, "gathered rows need candidates and num_candidates");
  if (p.k_quant != PKV_QUANT_NONE && !x.k_scale) return fail(PKV_EINVAL, "k_scale is NULL");
  if (p.layout == PKV_SEPARATE && p.v_quant != PKV_QUANT_NONE && !x.v_scale)
    return fail(PKV_EINVAL, "v_scale is NULL");
  if (p.layout == PKV_LATENT && x.v_scale && x.v_scale != x.k_scale)
    return fail(PKV_EINVAL, "LATENT: v_scale must be NULL or equal to k_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
    return fail(PKV_EINVAL, "softmax_scale must be finite and >= 0");
  if (!aligned(x.query, 16)) return fail(PKV_EALIGN, "query is not 16-byte aligned");
  if (!aligned(x.key_cache, 16)) return fail(PKV_EALIGN, "key_cache is not 16-byte aligned");
  if (x.value_cache && !aligned(x.value_cache, 16))
    return fail(PKV_EALIGN, "value_cache is not 16-byte aligned");
  for (const void* q : {(const void*)x.block_table, (const void*)x.seq_lens,
                        (const void*)x.candidates, (const void*)x.num_candidates})
    if (q && !aligned(q, 4)) return fail(PKV_EALIGN, "an int32 array is not 4-byte aligned");
  if (x.k_scale && !aligned(x.k_scale, p.k_quant == PKV_QUANT_PER_CHANNEL ? 16 : 4))
    return fail(PKV_EALIGN, "k_scale is not aligned");
  if (x.v_scale && !aligned(x.v_scale, p.v_quant == PKV_QUANT_PER_CHANNEL ? 16 : 4))
    return fail(PKV_EALIGN, "v_scale is not aligned");
  return PKV_OK;
}

pkv_status check_workspace(const pkv_geometry& g, const void* ws, size_t bytes) {
  if (!ws) return fail(PKV_EINVAL, "workspace is NULL");
  if (!aligned(ws, 16)) return fail(PKV_EALIGN, "workspace is not 16-byte aligned");
  if (bytes < g.workspace_bytes)
    return fail(PKV_EWORKSPACE, "workspace_bytes %zu < required %llu", bytes,
                (unsigned long long)g.workspace_bytes);
  return PKV_OK;
}

pkv_status check_outputs(const void* out, const float* lse, const float* sink) {
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (!aligned(out, 16)) return fail(PKV_EALIGN, "out is not 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(PKV_EALIGN, "lse_out is not 4-byte aligned");
  if (sink && !aligned(sink, 4)) return fail(PKV_EALIGN, "head_sink is not 4-byte aligned");
  return PKV_OK;
}

pkv::SplitArgs split_args(const pkv_problem& p, const pkv_geometry& g, const Ptrs& x,
                          float softmax_scale, void* workspace) {
  pkv::SplitArgs a;
  std::memset(&a, 0, sizeof(a));
  const uint64_t pairs = (uint64_t)p.num_rows * qtok_of(p) * p.num_heads;
  a.query = static_cast<const uint16_t*>(x.query);
  a.key_cache = static_cast<const uint8_t*>(x.key_cache);
  a.value_cache = static_cast<const uint8_t*>(x.value_cache);
  a.block_table = x.block_table;
  a.seq_lens = x.seq_lens;
  a.candidates = x.candidates;
  a.num_candidates = x.num_candidates;
  a.k_scale = x.k_scale;
  const bool latent = p.layout == PKV_LATENT;
  a.v_scale = latent ? x.k_scale : x.v_scale;
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = a.ws_acc + pairs * g.num_splits * p.v_head_size;
  a.rows = p.num_rows;
  a.heads = p.num_heads;
  a.kv_heads = p.num_kv_heads;
  a.group = p.num_heads / p.num_kv_heads;
  a.qtok = qtok_of(p);
  a.head_blocks = g.head_blocks;
  a.units_row = (int)units_row_of(p, g.kv_heads_per_cta);
  a.kvp = g.kv_heads_per_cta > 1 ? g.kv_heads_per_cta : 0;
  a.block_size = p.block_size;
  a.log2_block = __builtin_ctz((unsigned)p.block_size);
  a.max_blocks_per_row = p.max_blocks_per_row;
  a.num_pool_blocks = p.num_pool_blocks;
  a.max_candidates = p.max_candidates;
  a.num_splits = g.num_splits;
  a.min_chunk = g.min_chunk;
  a.target_ctas = g.target_ctas;
  a.grid_ctas = g.grid_x;
  {
    const int64_t cap_pos = positions_cap(p);
    a.static_chunk = std::max<int>(g.min_chunk,
                                   (int)((((cap_pos + g.num_splits - 1) / g.num_splits) + 15) / 16 * 16));
  }
  a.k_quant = p.k_quant;
  a.v_quant = latent ? p.k_quant : p.v_quant;
  a.v_scale_stride = latent ? p.head_size : p.v_head_size;
  a.score_scale = softmax_scale;
  a.window = p.sliding_window;
  a.softcap = p.softcap;
  a.inv_softcap = p.softcap > 0.0f ? 1.0f / p.softcap : 0.0f;
  a.v_mult = 1.0f / 16.0f;  // the kernels' probability tiles carry a factor 16
  return a;
}

pkv::CombineArgs combine_args(const pkv_problem& p, const pkv_geometry& g, const void* ws,
                              const float* sink, void* out, float* lse) {
  pkv::CombineArgs c;
  const uint64_t pairs = (uint64_t)p.num_rows * qtok_of(p) * p.num_heads;
  c.ws_acc = static_cast<const float*>(ws);
  c.ws_ml = c.ws_acc + pairs * g.num_splits * p.v_head_size;
  c.head_sink = sink;
  c.out = out;
  c.lse_out = lse;
  c.rows = p.num_rows * qtok_of(p);
  c.heads = p.num_heads;
  c.num_splits = g.num_splits;
  c.skip_empty = g.target_ctas > 0;
  return c;
}

// Static checks for the quantise-on-write call: only the cache description
// matters (no rows, heads or block tables are involved).
pkv_status check_write(const pkv_problem* p, int32_t tokens, const void* key, const void* value,
                       const int64_t* slots, const float* ks, const float* vs, const void* kc,
                       const void* vc) {
  if (!p) return fail(PKV_EINVAL, "problem is NULL");
  if (tokens < 0) return fail(PKV_EINVAL, "num_tokens < 0");
  if (p->num_kv_heads <= 0) return fail(PKV_EINVAL, "num_kv_heads must be positive");
  if (p->head_size <= 0 || p->v_head_size <= 0 || p->head_size % 8 || p->v_head_size % 8)
    return fail(PKV_EINVAL, "head sizes must be positive multiples of 8");
  if (p->block_size <= 0 || p->num_pool_blocks <= 0)
    return fail(PKV_EINVAL, "block_size and num_pool_blocks must be positive");
  if (p->cache_dtype != PKV_F16 && p->cache_dtype != PKV_I8 && p->cache_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_EINVAL, "cache_dtype must be PKV_F16, PKV_I8 or PKV_FP8_E4M3FN");
  if (p->layout != PKV_SEPARATE && p->layout != PKV_LATENT)
    return fail(PKV_EINVAL, "layout must be PKV_SEPARATE or PKV_LATENT");
  const bool latent = p->layout == PKV_LATENT;
  for (int q : {p->k_quant, p->v_quant})
    if (q < PKV_QUANT_NONE || q > PKV_QUANT_PER_CHANNEL)
      return fail(PKV_EINVAL, "quant must be NONE, PER_TENSOR or PER_CHANNEL");
  if (p->cache_dtype != PKV_F16) {
    if (p->k_quant == PKV_QUANT_NONE)
      return fail(PKV_EINVAL, "a quantised cache needs k_quant PER_TENSOR or PER_CHANNEL");
    if (!latent && p->v_quant == PKV_QUANT_NONE)
      return fail(PKV_EINVAL, "a quantised cache needs v_quant PER_TENSOR or PER_CHANNEL");
  }
  const int64_t chunks = (int64_t)p->num_kv_heads * ((p->head_size + (latent ? 0 : p->v_head_size)) / 8);
  if (chunks > INT32_MAX || (chunks * tokens + 255) / 256 > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "num_tokens * num_kv_heads * head sizes is too large");
  if (tokens > 0) {
    if (!key) return fail(PKV_EINVAL, "key is NULL");
    if (!slots) return fail(PKV_EINVAL, "slot_mapping is NULL");
  }
  if (!kc) return fail(PKV_EINVAL, "key_cache is NULL");
  if (latent && (value || vc))
    return fail(PKV_EINVAL, "value and value_cache must be NULL for the LATENT layout");
  if (!latent && !vc) return fail(PKV_EINVAL, "value_cache is NULL");
  if (!latent && tokens > 0 && !value) return fail(PKV_EINVAL, "value is NULL");
  if (p->k_quant != PKV_QUANT_NONE && !ks) return fail(PKV_EINVAL, "k_scale is NULL");
  if (!latent && p->v_quant != PKV_QUANT_NONE && !vs) return fail(PKV_EINVAL, "v_scale is NULL");
  for (const void* q : {key, value, kc, vc})
    if (q && !aligned(q, 16)) return fail(PKV_EALIGN, "a K/V array or cache is not 16-byte aligned");
  if (slots && !aligned(slots, 8)) return fail(PKV_EALIGN, "slot_mapping is not 8-byte aligned");
  if (ks && !aligned(ks, p->k_quant == PKV_QUANT_PER_CHANNEL ? 16 : 4))
    return fail(PKV_EALIGN, "k_scale is not aligned");
  if (!latent && vs && !aligned(vs, p->v_quant == PKV_QUANT_PER_CHANNEL ? 16 : 4))
    return fail(PKV_EALIGN, "v_scale is not aligned");
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// Workspace of paged_decode_attention_noalloc: a file-scope device array,
// one copy per GPU, that holds the split partials (the memory the caller
// passes as `workspace` to paged_decode_attention).  Host code never uses
// its name as an address: the device address of the current GPU's copy comes
// from hipGetSymbolAddress, once per device, and is cached.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_WORKSPACE_BYTES];

namespace {

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;

// Device address of the current device's scratch copy (resolved once per
// device, with that device current).
pkv_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(PKV_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: no kernel for this problem";
    case PKV_EALIGN: return "PKV_EALIGN: misaligned pointer";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE: workspace too small";
    case PKV_EHIP: return "PKV_EHIP: HIP runtime error";
    default: return "unknown pkv_status";
  }
}

const char* pkv_last_error(void) { return g_err; }

pkv_status split_geometry(const pkv_problem* problem, const pkv_geometry_opts* opts,
                          pkv_geometry* out) {
  g_err[0] = 0;
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  pkv_status st = check_problem(problem);
  if (st != PKV_OK) return st;
  const pkv_problem& p = *problem;
  pkv_geometry_opts o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.num_cus < 0 || o.ctas_per_cu < 0 || o.splits_override < 0 || o.min_chunk < 0 ||
      o.max_splits < 0 || o.waves < 0)
    return fail(PKV_EINVAL, "geometry options must be >= 0");
  const bool gathered = p.max_candidates > 0;
  if (o.min_chunk % 16) return fail(PKV_EINVAL, "min_chunk must be a multiple of 16");
  const int max_splits = o.max_splits ? o.max_splits : pkv::kMaxSplits;
  if (max_splits > pkv::kMaxSplits)
    return fail(PKV_EINVAL, "max_splits %d exceeds %d", max_splits, pkv::kMaxSplits);
  const int waves_req = o.waves;

  const int head_blocks = ceil_div(vgroup_of(p), 16);
  // KV heads per CTA: four when the problem allows it (whole-record reads),
  // unless the caller asks for one
  if (o.kv_heads_per_cta != 0 && o.kv_heads_per_cta != 1 && o.kv_heads_per_cta != pkv::kKvHeadsPerCta &&
      o.kv_heads_per_cta != pkv::kKvHeadsPerCtaWide)
    return fail(PKV_EINVAL, "kv_heads_per_cta must be 0, 1, %d or %d", pkv::kKvHeadsPerCta,
                pkv::kKvHeadsPerCtaWide);
  if (o.kv_heads_per_cta > 1 && !kvp_allowed(p, o.kv_heads_per_cta))
    return fail(PKV_EUNSUPPORTED, "%d KV heads per CTA need dense rows, the SEPARATE layout, a "
                                  "multiple of %d KV heads and at most 16 head slots per KV head "
                                  "(32 with 4 KV heads per CTA and head size up to 128)",
                o.kv_heads_per_cta, o.kv_heads_per_cta);
  // (automatic for head sizes up to 128: measured faster there; larger
  // heads need more registers per wave than two waves per SIMD allow.  With
  // 17-32 head slots per KV head: for FP16 caches, and for one-byte codes
  // with several query tokens per row -- C3's lengths, 8 tokens: INT8 56.2
  // against 59.7 us, FP8 54.5 against 58.1 -- but not for one-byte codes
  // with one token and 20 or 32 query heads per KV head, where one KV head
  // per CTA stayed faster: 36.3 against 37.0 us, 38.5 against 39.9)
  const bool auto_kvp = kvp_allowed(p, pkv::kKvHeadsPerCta) && p.head_size <= 128 &&
                        (vgroup_of(p) <= 16 || p.cache_dtype == PKV_F16 || qtok_of(p) > 1);
  const int kv_per_cta = o.kv_heads_per_cta ? o.kv_heads_per_cta : (auto_kvp ? pkv::kKvHeadsPerCta : 1);
  const pkv::Variant var = variant_for(p, kv_per_cta);
  const int64_t units = std::max<int64_t>(1, (int64_t)p.num_rows * units_row_of(p, kv_per_cta));
  const int64_t cap = positions_cap(p);

  // The device balances chunk sizes across rows from the live lengths when
  // the row count is modest (each CTA reads every row's length).
  if (o.balance < 0 || o.balance > 2) return fail(PKV_EINVAL, "balance must be 0, 1 or 2");
  // (its CTAs sum the live positions of all rows in 32 bits: only when that
  // sum cannot reach 2^31)
  bool balanced = balance_fits(p) &&
                  (o.balance == 1 || (o.balance == 0 && p.num_rows >= kMinBalancedRows));
  // Several KV heads per CTA with several query tokens per row, or with two
  // head blocks per wave (17-32 head slots per KV head): all CTAs resident
  // in one round (see target below), one CTA per CU (FP16 caches, and any
  // cache with one head block), and for two head blocks the quarter-partial
  // chunk floor on FP16-sized KV bytes.  Measured on MI355X with C3's
  // lengths against the plain four-KV-head geometry (two CTAs per CU): 2, 3
  // and 4 tokens per row 63.8 -> 61.3, 66.8 -> 63.4, 68.7 -> 64.5 us, INT8
  // with 4 tokens 48.6 -> 45.9 us; against one KV head per CTA: 8 tokens
  // 92.5 -> 79.2 us, 32 query heads per KV head 53.8 -> 46.4 us, 20 heads
  // 50.2 -> 41.7 us (two CTAs per CU, a partial second round or the
  // eighth-partial floor left tails; with one token per row C3 itself gains
  // nothing from it).  With two head blocks and one-byte codes two CTAs per
  // CU measured faster (C3 with 8 tokens, INT8: 56.2 against 67.1 us; FP8,
  // whose kernel fits three per CU: 54.5 against 61.3 us at three).
  const bool two_blocks = var.vb == 2;
  const bool one_round = var.kvp > 0 && (two_blocks || var.mt);
  const bool one_per_cu = one_round && (!two_blocks || p.cache_dtype == PKV_F16);
  int cus = o.num_cus, occ = o.ctas_per_cu;
  if (cus == 0 || occ == 0) {
    int qc = 0, qo = 0;
    st = device_numbers(var, &qc, occ == 0 ? &qo : nullptr);
    if (st != PKV_OK) return st;
    if (cus == 0) cus = qc;
    if (occ == 0) occ = one_per_cu ? 1 : (two_blocks ? std::min(qo, 2) : qo);
  }
  // Live-balanced mode: about two rounds of CTAs per resident slot let the
  // dispatcher even out what per-row rounding leaves (measured on MI355X),
  // unless a split's partial (written once, read once by the combine) is at
  // least half the KV bytes of a min_chunk -- then halving the chunk costs
  // more traffic than it saves (latent rows: 16 heads x 512 FP32 per split).
  // (per work unit: its KV heads' query heads, and the KV bytes of one
  // position of all its KV heads)
  const int64_t partial_bytes =
      (int64_t)kv_per_cta * vgroup_of(p) * (p.v_head_size + 2) * 4;
  const int64_t row_bytes = (int64_t)kv_per_cta *
                            (p.layout == PKV_LATENT ? p.head_size : p.head_size + p.v_head_size) *
                            (p.cache_dtype == PKV_F16 ? 2 : 1);
  // Automatic chunk floor: 64 positions, raised to the power of two that
  // keeps a split's partial (written once, read back once by the combine) at
  // most an eighth of the KV bytes it covers while the grid still gives
  // every CU a CTA (two CTAs with several KV heads per CTA: the PagedAttention
  // page's 1024 x 32 and 4096 x 8 INT8 shapes 18.5 -> 15.9 and 18.8 -> 16.3
  // us with the quarter floor below instead); else at most a quarter while it
  // still fills a quarter of the resident CTAs; else 64 (a small step is
  // bound by latency, and more, shorter splits finish sooner).  With two head blocks per wave: at
  // most a quarter of the bytes the positions would take in FP16, always.
  int min_chunk = o.min_chunk;
  if (min_chunk == 0) {
    min_chunk = 64;
    auto floor_for = [&](int64_t frac, int64_t rb) {
      int64_t c = 16;
      while (c < ceil_div(frac * partial_bytes, rb)) c *= 2;
      return std::min<int64_t>(c, 1 << 20);
    };
    const int64_t c8 = floor_for(8, row_bytes), c4 = floor_for(4, row_bytes);
    if (two_blocks)
      min_chunk = (int)std::max<int64_t>(
          min_chunk, floor_for(4, row_bytes * (p.cache_dtype == PKV_F16 ? 1 : 2)));
    else if (c8 > min_chunk && units * ceil_div(cap, c8) >= (int64_t)cus * (kv_per_cta > 1 ? 2 : 1))
      min_chunk = (int)c8;
    else if (c4 > min_chunk && units * ceil_div(cap, c4) * 4 >= (int64_t)cus * occ)
      min_chunk = (int)c4;
  }
  // The live-balanced decomposition cannot cut the rows finer than the
  // static one when even full rows would get the chunk floor (rows x cap x
  // units per row <= resident CTAs x min_chunk: both then cut every row into
  // the same min_chunk pieces), and it reads all row lengths before the
  // first block-id read; so automatic mode takes the static one there
  // (measured on MI355X, latent C5: 24.4 against 25.3 us; with lengths
  // U[1024, 4096] 23.9 against 24.1).
  if (balanced && o.balance == 0 &&
      (int64_t)p.num_rows * cap * units_row_of(p, kv_per_cta) <= (int64_t)cus * occ * min_chunk)
    balanced = false;
  const bool cheap_partials = 2 * partial_bytes < row_bytes * min_chunk;
  // (four KV heads per CTA: one round; their CTAs already carry four
  // units' partials, and a second round measured slower)
  const int waves = waves_req ? waves_req
                              : (balanced && cheap_partials && kv_per_cta == 1 ? 2 : 1);
  int64_t target = (int64_t)waves * cus * occ;
  // (per-row rounding adds at most one CTA per unit to the live-balanced
  // count: in the one-round cases above, leave that room in the round)
  if (one_round && balanced && 2 * units <= target) target -= units;
  int S;
  if (o.splits_override > 0) {
    S = o.splits_override;
  } else {
    if (gathered) {
      // 64-candidate tiles; smallest power-of-two tiles per split for which
      // all tiles of all units fit the target number of CTAs.
      const int64_t tiles = (cap + 63) / 64;
      int64_t tps = 1;
      while ((ceil_div(tiles, tps) * units > target || 64 * tps < min_chunk) && tps < tiles) tps *= 2;
      S = ceil_div(tiles, tps);
    } else {
      // live-balanced chunks: leave room for rows up to 4x the mean work
      const int64_t want = balanced ? 4 * target : target;
      S = (int)std::min<int64_t>(ceil_div(want, units), ceil_div(cap, min_chunk));
    }
  }
  // Short rows take one split (with the automatic split count and chunk
  // floor): at most 256 positions per row is four 16-token tiles per wave of
  // a CTA, and one launch with the direct output beats the split kernel plus
  // the combine's second launch (measured on MI355X with one row, 4q/1kv,
  // head 64: 128 positions 4.5 against 5.7 us at 2 splits, 256 positions
  // 5.3 against 6.1 at 4; at 512 positions 8 splits win, 6.6 against 7.1).
  if (o.splits_override == 0 && o.min_chunk == 0 && cap <= kOneSplitCap) S = 1;
  S = std::max(1, std::min(S, max_splits));
  S = std::max(1, std::min<int>(S, ceil_div(cap, 16)));

  out->num_splits = S;
  out->min_chunk = min_chunk;
  out->threads = pkv::threads_of(var);
  out->head_blocks = head_blocks;
  out->target_ctas = balanced ? (int32_t)std::min<int64_t>(target, INT32_MAX) : 0;
  out->kv_heads_per_cta = kv_per_cta;
  const int64_t grid = grid_ctas_for(p, S, out->target_ctas, kv_per_cta);
  if (grid > INT32_MAX) return fail(PKV_EUNSUPPORTED, "too many CTAs (%lld)", (long long)grid);
  out->grid_x = (int32_t)grid;
  out->grid_y = 1;
  out->grid_z = 1;
  out->workspace_bytes = workspace_bytes_for(p, S);
  return PKV_OK;
}

pkv_status paged_decode_partials(const pkv_problem* problem, const pkv_geometry* geometry,
                                 const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* candidates,
                                 const int32_t* num_candidates, const float* k_scale,
                                 const float* v_scale, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  pkv_status st = check_problem(problem);
  if (st != PKV_OK) return st;
  st = check_geometry(*problem, geometry);
  if (st != PKV_OK) return st;
  const Ptrs x{query, key_cache, value_cache, block_table, seq_lens,
               candidates, num_candidates, k_scale, v_scale};
  st = check_inputs(*problem, x, softmax_scale);
  if (st != PKV_OK) return st;
  st = check_workspace(*geometry, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (problem->num_rows == 0) return PKV_OK;
  const pkv::SplitArgs a = split_args(*problem, *geometry, x, softmax_scale, workspace);
  return hip_status(pkv::launch_split(variant_of(*problem), a, static_cast<hipStream_t>(stream)),
                    "split kernel launch");
}

pkv_status split_combine(const pkv_problem* problem, const pkv_geometry* geometry,
                         const void* workspace, size_t workspace_bytes, const float* head_sink,
                         void* out, float* lse_out, void* stream) {
  g_err[0] = 0;
  pkv_status st = check_problem(problem);
  if (st != PKV_OK) return st;
  st = check_geometry(*problem, geometry);
  if (st != PKV_OK) return st;
  st = check_workspace(*geometry, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  st = check_outputs(out, lse_out, head_sink);
  if (st != PKV_OK) return st;
  if (problem->num_rows == 0) return PKV_OK;
  const pkv::CombineArgs c = combine_args(*problem, *geometry, workspace, head_sink, out, lse_out);
  return hip_status(pkv::launch_combine(problem->v_head_size, problem->out_dtype, c,
                                        static_cast<hipStream_t>(stream)),
                    "combine kernel launch");
}

pkv_status paged_decode_attention(const pkv_problem* problem, const pkv_geometry* geometry,
                                  const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* candidates,
                                  const int32_t* num_candidates, const float* k_scale,
                                  const float* v_scale, float softmax_scale,
                                  const float* head_sink, void* out, float* lse_out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  pkv_status st = check_problem(problem);
  if (st != PKV_OK) return st;
  st = check_geometry(*problem, geometry);
  if (st != PKV_OK) return st;
  const Ptrs x{query, key_cache, value_cache, block_table, seq_lens,
               candidates, num_candidates, k_scale, v_scale};
  st = check_inputs(*problem, x, softmax_scale);
  if (st != PKV_OK) return st;
  st = check_workspace(*geometry, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  st = check_outputs(out, lse_out, head_sink);
  if (st != PKV_OK) return st;
  if (problem->num_rows == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pkv::SplitArgs a = split_args(*problem, *geometry, x, softmax_scale, workspace);
  if (geometry->num_splits == 1) {
    // one split per row: the split kernel writes the output itself (exactly
    // what the combine would), and there is no second launch
    a.direct = 1;
    a.out_f32 = problem->out_dtype == PKV_F32;
    a.out = out;
    a.lse_out = lse_out;
    a.head_sink = head_sink;
    return hip_status(pkv::launch_split(variant_of(*problem), a, s), "split kernel launch");
  }
  st = hip_status(pkv::launch_split(variant_of(*problem), a, s), "split kernel launch");
  if (st != PKV_OK) return st;
  const pkv::CombineArgs c = combine_args(*problem, *geometry, workspace, head_sink, out, lse_out);
  return hip_status(pkv::launch_combine(problem->v_head_size, problem->out_dtype, c, s),
                    "combine kernel launch");
}

pkv_status paged_decode_attention_noalloc(const pkv_problem* problem,
                                          const pkv_geometry* geometry, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const int32_t* candidates,
                                          const int32_t* num_candidates, const float* k_scale,
                                          const float* v_scale, float softmax_scale,
                                          const float* head_sink, void* out, float* lse_out,
                                          void* stream) {
  g_err[0] = 0;
  pkv_status st = check_problem(problem);
  if (st != PKV_OK) return st;
  st = check_geometry(*problem, geometry);
  if (st != PKV_OK) return st;
  if (geometry->workspace_bytes > (uint64_t)PKV_NOALLOC_WORKSPACE_BYTES)
    return fail(PKV_EWORKSPACE,
                "the problem needs %llu bytes of workspace, more than the %llu bytes the "
                "allocation-free entry point holds per device (fewer rows or splits fit)",
                (unsigned long long)geometry->workspace_bytes,
                (unsigned long long)PKV_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != PKV_OK) return st;
  return paged_decode_attention(problem, geometry, query, key_cache, value_cache, block_table,
                                seq_lens, candidates, num_candidates, k_scale, v_scale,
                                softmax_scale, head_sink, out, lse_out, ws,
                                (size_t)PKV_NOALLOC_WORKSPACE_BYTES, stream);
}

pkv_status reshape_and_cache(const pkv_problem* problem, int32_t num_tokens, const void* key,
                             const void* value, const int64_t* slot_mapping,
                             const float* k_scale, const float* v_scale, void* key_cache,
                             void* value_cache, void* stream) {
  g_err[0] = 0;
  const pkv_status st = check_write(problem, num_tokens, key, value, slot_mapping, k_scale,
                                    v_scale, key_cache, value_cache);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  const pkv_problem& p = *problem;
  const bool latent = p.layout == PKV_LATENT;
  pkv::WriteArgs a{};
  a.key = static_cast<const uint16_t*>(key);
  a.value = latent ? nullptr : static_cast<const uint16_t*>(value);
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = latent ? nullptr : v_scale;
  a.key_cache = static_cast<uint8_t*>(key_cache);
  a.value_cache = latent ? nullptr : static_cast<uint8_t*>(value_cache);
  a.n_slots = (int64_t)p.num_pool_blocks * p.block_size;
  a.tokens = num_tokens;
  a.kv_heads = p.num_kv_heads;
  a.head_size = p.head_size;
  a.v_head_size = p.v_head_size;
  a.chunks_k = p.head_size / 8;
  a.chunks_v = latent ? 0 : p.v_head_size / 8;
  a.k_quant = p.k_quant;
  a.v_quant = latent ? PKV_QUANT_NONE : p.v_quant;
  return hip_status(pkv::launch_cache_write(p.cache_dtype, a, static_cast<hipStream_t>(stream)),
                    "cache write launch");
}

}  // extern "C"
