/* A plain C11 consumer of the C ABI: compiles against include/pkv.h with a C
 * compiler (no C++), links libpkv.so, and prints the geometry of a
 * continuous-batching FP16 problem (16 rows, 32 query / 8 KV heads, head 128,
 * block 16, 512 blocks per row) for a given CU count and occupancy, then the
 * status and message of a rejected problem.  No kernel runs. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

int main(void) {
  pkv_problem p;
  memset(&p, 0, sizeof p);
  p.num_rows = 16;
  p.num_heads = 32;
  p.num_kv_heads = 8;
  p.head_size = 128;
  p.v_head_size = 128;
  p.block_size = 16;
  p.max_blocks_per_row = 512;
  p.num_pool_blocks = 5000;
  p.cache_dtype = PKV_F16;
  p.out_dtype = PKV_F16;
  p.k_quant = PKV_QUANT_NONE;
  p.v_quant = PKV_QUANT_NONE;
  p.layout = PKV_SEPARATE;
  p.query_tokens = 1;

  pkv_geometry_opts o;
  memset(&o, 0, sizeof o);
  o.num_cus = 256;
  o.ctas_per_cu = 2;

  pkv_geometry g;
  pkv_status st = split_geometry(&p, &o, &g);
  printf("status=%d\n", (int)st);
  if (st != PKV_OK) return 1;
  printf("num_splits=%d\nmin_chunk=%d\nthreads=%d\nhead_blocks=%d\ngrid_x=%d\ntarget_ctas=%d\n"
         "kv_heads_per_cta=%d\nworkspace_bytes=%llu\n",
         g.num_splits, g.min_chunk, g.threads, g.head_blocks, g.grid_x, g.target_ctas,
         g.kv_heads_per_cta, (unsigned long long)g.workspace_bytes);

  p.num_heads = 30; /* not a multiple of num_kv_heads */
  st = split_geometry(&p, &o, &g);
  printf("bad_status=%d\nbad_name=%s\nbad_message=%s\n", (int)st, pkv_status_string(st),
         pkv_last_error());
  return st == PKV_EINVAL ? 0 : 2;
}
