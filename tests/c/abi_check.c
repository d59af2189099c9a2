/* A plain C11 client of the library's C ABI (built and run by test_c_abi.py).
 * It only calls size queries and calls that fail host validation, so it needs
 * no GPU: every line it prints is checked by the test. */
#include <stdio.h>
#include <string.h>

#include "kvtc.h"

int main(void) {
  const int32_t rk[2] = {64, 32}, bk[2] = {4, 8}, rv[2] = {128, 64}, bv[2] = {2, 4};
  kv_layout lay;
  memset(&lay, 0, sizeof lay);
  lay.head_dim = 128;
  lay.n_kv_heads = 2;
  lay.n_q_heads = 8;
  lay.batch = 3;
  lay.capacity = 1000;
  lay.rank_k = rk;
  lay.bits_k = bk;
  lay.rank_v = rv;
  lay.bits_v = bv;

  printf("record_words %d %d %d\n", kv_record_words(64, 4), kv_record_words(16, 6), kv_record_words(48, 4));

  size_t kb = 0, vb = 0;
  const kv_status sk = kv_cache_bytes(&lay, 0, &kb), sv = kv_cache_bytes(&lay, 1, &vb);
  printf("cache_bytes %d %zu %d %zu\n", (int)sk, kb, (int)sv, vb);

  int32_t cls = -9, splits = -9, wgs = -9;
  const kv_status sp = kv_attend_plan(&lay, 1000, 0, &cls, &splits, &wgs);
  printf("plan %d %d %d %d\n", (int)sp, cls, splits, wgs);

  /* null query: rejected on the host before any launch */
  const kv_status sa = kv_attend_decode(&lay, NULL, KV_F16, 1000, NULL, NULL, NULL, NULL, 0.088f, NULL, NULL, 0,
                                        NULL);
  const char *msg = kv_last_error();
  printf("attend_null %d %d\n", (int)sa, msg != NULL && msg[0] != '\0');

  /* unsupported head dimension */
  lay.head_dim = 64;
  const kv_status su = kv_cache_bytes(&lay, 0, &kb);
  printf("head_dim_64 %d\n", (int)su);
  return 0;
}
