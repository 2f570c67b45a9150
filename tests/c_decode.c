/* A plain C11 program that runs decode steps through the C ABI on the GPU,
 * with device memory from the HIP runtime's C API (no C++, no PyTorch), on
 * a problem whose result has a closed form.  The query is zero, so every
 * score is 0 and every probability 1: output channel c of query head h is
 * the mean of the row's value codes in channel c of KV head h / group,
 * times v_scale, and lse = log(len).  Rows of 1, 100 and 128 tokens over
 * reversed, interleaved block tables; INT8 per-tensor caches; FP32 output;
 * the automatic geometry and three splits.  A too-small workspace must be
 * refused with PKV_EWORKSPACE.  Prints "ok" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pkv.h"

#define HIP_OK(x)                                                           \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 3;                                                             \
    }                                                                       \
  } while (0)

enum { ROWS = 3, HEADS = 8, KVH = 2, GROUP = HEADS / KVH, D = 64, B = 16, MBPR = 8 };
enum { POOL = ROWS * MBPR, SLOT_ELEMS = KVH * D, CACHE_ELEMS = POOL * B * SLOT_ELEMS };

static int8_t kc[CACHE_ELEMS], vc[CACHE_ELEMS];
static uint16_t q[ROWS * HEADS * D]; /* FP16 +0 */
static float out[ROWS * HEADS * D], lse[ROWS * HEADS];

static int code_of(int slot, int g, int c, int salt) {
  return (slot * 7 + g * 5 + c * 3 + salt) % 255 - 127;
}

/* pool block of row r's j-th logical block: rows interleaved, order reversed */
static int block_of(int r, int j) { return (MBPR - 1 - j) * ROWS + r; }

static int run(const pkv_problem* p, const pkv_geometry_opts* o, const int32_t* lens,
               const void* dq, const void* dk, const void* dv, const int32_t* dbt,
               const int32_t* dlens, const float* dks, const float* dvs, float vs, void* dout,
               float* dlse) {
  pkv_geometry g;
  pkv_status st = split_geometry(p, o, &g);
  if (st != PKV_OK) {
    fprintf(stderr, "split_geometry: %s %s\n", pkv_status_string(st), pkv_last_error());
    return 4;
  }
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, (size_t)g.workspace_bytes));
  st = paged_decode_attention(p, &g, dq, dk, dv, dbt, dlens, NULL, NULL, dks, dvs, 0.125f, NULL,
                              dout, dlse, ws, (size_t)g.workspace_bytes, NULL);
  if (st != PKV_OK) {
    fprintf(stderr, "paged_decode_attention: %s %s\n", pkv_status_string(st), pkv_last_error());
    return 5;
  }
  if (g.workspace_bytes > 16) {
    st = paged_decode_attention(p, &g, dq, dk, dv, dbt, dlens, NULL, NULL, dks, dvs, 0.125f,
                                NULL, dout, dlse, ws, 16, NULL);
    if (st != PKV_EWORKSPACE) {
      fprintf(stderr, "a 16-byte workspace gave status %d\n", (int)st);
      return 6;
    }
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));
  HIP_OK(hipFree(ws));
  for (int r = 0; r < ROWS; ++r)
    for (int h = 0; h < HEADS; ++h) {
      const int g_kv = h / GROUP;
      const double want_lse = log((double)lens[r]);
      if (fabs(lse[r * HEADS + h] - want_lse) > 1e-6 * (1.0 + want_lse)) {
        fprintf(stderr, "lse row %d head %d: %.9g, want %.9g\n", r, h, lse[r * HEADS + h],
                want_lse);
        return 7;
      }
      for (int c = 0; c < D; ++c) {
        double sum = 0.0;
        for (int t = 0; t < lens[r]; ++t) {
          const int slot = block_of(r, t / B) * B + t % B;
          sum += code_of(slot, g_kv, c, 1);
        }
        const double want = (double)vs * sum / lens[r];
        const double got = out[(r * HEADS + h) * D + c];
        if (fabs(got - want) > 1e-6 * (1.0 + fabs(want))) {
          fprintf(stderr, "out row %d head %d channel %d: %.9g, want %.9g (S=%d)\n", r, h, c,
                  got, want, g.num_splits);
          return 8;
        }
      }
    }
  printf("num_splits=%d checked\n", g.num_splits);
  return 0;
}

int main(void) {
  pkv_problem p;
  memset(&p, 0, sizeof p);
  p.num_rows = ROWS;
  p.num_heads = HEADS;
  p.num_kv_heads = KVH;
  p.head_size = D;
  p.v_head_size = D;
  p.block_size = B;
  p.max_blocks_per_row = MBPR;
  p.num_pool_blocks = POOL;
  p.cache_dtype = PKV_I8;
  p.out_dtype = PKV_F32;
  p.k_quant = PKV_QUANT_PER_TENSOR;
  p.v_quant = PKV_QUANT_PER_TENSOR;
  p.layout = PKV_SEPARATE;
  p.query_tokens = 1;

  const int32_t lens[ROWS] = {1, 100, 128};
  int32_t bt[ROWS * MBPR];
  for (int r = 0; r < ROWS; ++r)
    for (int j = 0; j < MBPR; ++j) bt[r * MBPR + j] = block_of(r, j);
  for (int slot = 0; slot < POOL * B; ++slot)
    for (int g = 0; g < KVH; ++g)
      for (int c = 0; c < D; ++c) {
        kc[(slot * KVH + g) * D + c] = (int8_t)code_of(slot, g, c, 0);
        vc[(slot * KVH + g) * D + c] = (int8_t)code_of(slot, g, c, 1);
      }
  const float ks = 0.01f, vs = 0.02f;

  void *dq, *dk, *dv, *dout;
  int32_t *dbt, *dlens;
  float *dks, *dvs, *dlse;
  HIP_OK(hipMalloc(&dq, sizeof q));
  HIP_OK(hipMalloc(&dk, sizeof kc));
  HIP_OK(hipMalloc(&dv, sizeof vc));
  HIP_OK(hipMalloc((void**)&dbt, sizeof bt));
  HIP_OK(hipMalloc((void**)&dlens, sizeof lens));
  HIP_OK(hipMalloc((void**)&dks, sizeof ks));
  HIP_OK(hipMalloc((void**)&dvs, sizeof vs));
  HIP_OK(hipMalloc(&dout, sizeof out));
  HIP_OK(hipMalloc((void**)&dlse, sizeof lse));
  HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, kc, sizeof kc, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, vc, sizeof vc, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dbt, bt, sizeof bt, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dks, &ks, sizeof ks, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dvs, &vs, sizeof vs, hipMemcpyHostToDevice));

  pkv_geometry_opts o;
  memset(&o, 0, sizeof o);
  int rc = run(&p, &o, lens, dq, dk, dv, dbt, dlens, dks, dvs, vs, dout, dlse);
  if (rc) return rc;
  o.splits_override = 3;
  o.min_chunk = 16;
  rc = run(&p, &o, lens, dq, dk, dv, dbt, dlens, dks, dvs, vs, dout, dlse);
  if (rc) return rc;

  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dbt));
  HIP_OK(hipFree(dlens));
  HIP_OK(hipFree(dks));
  HIP_OK(hipFree(dvs));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dlse));
  printf("ok\n");
  return 0;
}
