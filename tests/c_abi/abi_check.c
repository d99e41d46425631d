/* Host-only use of the C ABI from plain C99: every call below is rejected by
 * the library's host-side validation before any HIP call, so no GPU is
 * needed.  Prints "ok" and exits 0 when every status is the expected one. */
#include <stdio.h>
#include <string.h>

#include "qsakv.h"

static int fails = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    printf("%s: got %d (%s), want %d (%s)\n", what, got, qkv_status_str(got), want,
           qkv_status_str(want));
    ++fails;
  }
}

int main(void) {
  qkv_cache c;
  qsa_args a;
  qkv_calib_result r;
  size_t kb = 0, vb = 0, sb = 0;
  void *dummy = (void *)(size_t)0x10000;

  expect("abi version", qkv_abi_version(), QSAKV_ABI_VERSION);
  expect("cache bytes", qkv_cache_bytes(QKV_CACHE_INT8, 4, 64, 2, 256, &kb, &vb, &sb), QKV_OK);
  if (kb != (size_t)4 * 64 * 2 * 256 || sb != (size_t)4 * 64 * 2 * 2 * 4) ++fails;

  memset(&c, 0, sizeof c);
  c.kind = QKV_CACHE_E4M3;
  c.num_blocks = 4;
  c.block_size = 64;
  c.num_kv_heads = 2;
  c.head_dim = 256;
  c.k = c.v = dummy;
  c.k_scale = 0.0f;                 /* fails closed */
  c.v_scale = 1.0f;
  memset(&a, 0, sizeof a);
  a.q = dummy;
  a.q_dtype = QKV_FP16;
  a.num_rows = 1;
  a.num_q_heads = 16;
  a.num_seqs = 1;
  a.row_seq = a.block_table = a.topk_idx = (const int32_t *)dummy;
  a.block_table_stride = 4;
  a.topk = 8;
  a.sm_scale = 0.0625f;
  a.out_dtype = QKV_FP16;
  a.out = dummy;
  expect("e4m3 zero scale", qsa_sparse_attn_prefill(&c, &a, NULL), QKV_ERR_BAD_SCALE);
  expect("null cache", qsa_sparse_attn_prefill(NULL, &a, NULL), QKV_ERR_NULL);
  c.k_scale = 1.0f;                 /* legal from here on */
  expect("decode splits", qsa_sparse_attn_decode(&c, &a, 0, dummy, 1 << 20, NULL),
         QKV_ERR_UNSUPPORTED);
  expect("write negative tokens",
         kv_quant_write(&c, dummy, dummy, QKV_FP16, -1, (const int64_t *)dummy, NULL),
         QKV_ERR_BAD_SHAPE);
  expect("calib bad scale", kv_calib_stats(dummy, QKV_FP16, 16, -1.0f, &r, dummy,
                                           qkv_calib_workspace_bytes(), NULL),
         QKV_ERR_BAD_SCALE);
  expect("topk no k", qsa_topk_select(dummy, QKV_FP32, 4, 1024, (const int32_t *)dummy, 0,
                                      (int32_t *)dummy, NULL, 0, NULL),
         QKV_ERR_BAD_SHAPE);
  expect("topk no rows", qsa_topk_select(NULL, QKV_FP16, 0, 0, NULL, 1, NULL, NULL, 0, NULL),
         QKV_OK);
  /* the no-alloc decode: the same argument checks, then its scratch limit
     (40 rows x 16 heads x 64 splits x 256 floats is 40 MiB > 16 MiB) */
  expect("noalloc splits", qsa_sparse_attn_decode_noalloc(&c, &a, 65, NULL),
         QKV_ERR_UNSUPPORTED);
  a.num_rows = 40;
  a.num_q_heads = 16;
  expect("noalloc oversize", qsa_sparse_attn_decode_noalloc(&c, &a, 64, NULL), QKV_ERR_SCRATCH);
  a.num_rows = 0;
  expect("noalloc no rows", qsa_sparse_attn_decode_noalloc(&c, &a, 8, NULL), QKV_OK);
  a.num_rows = 1;
  if (qsa_topk_workspace_bytes(40, 131072, 2048) == 0) ++fails;
  if (qsa_decode_workspace_bytes(40, 16, 256, 8) == 0) ++fails;
  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
