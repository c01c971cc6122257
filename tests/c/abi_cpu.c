/* The C ABI from plain C, without a GPU: descriptor checks and layout queries.
 * Built and run by tests/test_c_programs.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hc.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #c, hc_last_error()); \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main(void) {
  void* layers[32];
  for (int l = 0; l < 32; l++) layers[l] = (void*)(uintptr_t)(0x10000 * (l + 1));
  hc_pool_desc d;
  memset(&d, 0, sizeof(d));
  d.num_layers = 32;
  d.page_size = 64;
  d.num_subbufs = 2;
  d.layout = HC_LAYOUT_PAGE_FIRST;
  for (int b = 0; b < 2; b++) {
    d.sub[b].granularity = HC_TOKEN_ROWS;
    d.sub[b].elem_bytes = 2048;
    d.sub[b].device_layers = layers;
  }
  d.device_slots = 262144;
  d.host_pages = 8192;
  d.host_base = (void*)(uintptr_t)0x7f0000000000ull;
  d.host_bytes = (int64_t)1 << 40;
  CHECK(hc_desc_check(&d) == HC_OK);
  int64_t v = 0;
  CHECK(hc_host_pool_bytes(&d, &v) == HC_OK && v == 68719476736ll);
  CHECK(hc_host_offset(&d, 1, 8191, 31, 63, &v) == HC_OK && v == 68719474688ll);
  CHECK(hc_staging_page_bytes(&d, &v) == HC_OK && v == 8388608ll);
  d.layout = HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR;
  CHECK(hc_host_offset(&d, 0, 3, 5, 7, &v) == HC_OK && v == 13051904ll);
  d.layout = HC_LAYOUT_KV_SPLIT_SHARD;
  d.shard_align = 4096;
  d.num_layers = 3;
  d.page_size = 16;
  d.sub[0].elem_bytes = 1024;
  d.sub[1].elem_bytes = 128;
  d.host_pages = 8;
  CHECK(hc_staging_page_bytes(&d, &v) == HC_OK && v == 57344);
  CHECK(hc_host_offset(&d, 1, 2, 1, 5, &v) == HC_OK && v == 166528);
  d.sub[1].elem_bytes = 100;
  CHECK(hc_desc_check(&d) == HC_ERR_UNSUPPORTED);
  CHECK(strstr(hc_last_error(), "multiple of 16") != NULL);
  CHECK(hc_pool_destroy(NULL) == HC_OK);
  CHECK(hc_load_back_layer(NULL, 0, NULL, NULL, 0, NULL) == HC_ERR_INVALID);
  uint64_t fp = 0;
  d.sub[1].elem_bytes = 128;
  CHECK(hc_cache_fingerprint(&d, "m", 1, &fp) == HC_OK && fp != 0);
  printf("abi_cpu ok (version %d)\n", hc_version());
  return 0;
}
