/* Oracle for the HiCache host<->device KV page transfer -- TEST INFRASTRUCTURE.
 * Declarations of hc_oracle.c for C test programs; see that file for what each
 * function computes and which passage of the pages it follows. */
#ifndef HC_ORACLE_H
#define HC_ORACLE_H
#include <stdint.h>

#define ORC_MAX_SUB 4
enum { ORC_OK = 0, ORC_ERR_INVALID = -1 };
enum { ORC_TOKEN_ROWS = 0, ORC_PAGE_BLOCKS = 1 };
enum { ORC_PAGE_FIRST = 0, ORC_KV_SPLIT_SHARD = 1, ORC_PAGE_FIRST_TOKEN_MAJOR = 2 };

typedef struct orc_geom {
  int32_t layers;
  int32_t page_size;
  int32_t nsub;
  int32_t layout;
  int64_t host_pages;
  int64_t device_slots;
  int64_t align;
  int32_t gran[ORC_MAX_SUB];
  int64_t bytes[ORC_MAX_SUB];
} orc_geom;

int64_t orc_sub_page_bytes(const orc_geom* g, int b);
int64_t orc_page_payload_bytes(const orc_geom* g);
int64_t orc_shard_bytes(const orc_geom* g);
int64_t orc_host_pool_bytes(const orc_geom* g);
int64_t orc_host_offset(const orc_geom* g, int b, int64_t p, int32_t l, int32_t r);
int64_t orc_device_offset(const orc_geom* g, int b, int64_t s);
int orc_check_geom(const orc_geom* g);
int orc_check_indices(const orc_geom* g, const int64_t* d, const int64_t* h, int64_t n);
int orc_write_back(const orc_geom* g, uint8_t* const* dev, uint8_t* host, const int64_t* d, const int64_t* h, int64_t n);
int orc_load_back_layer(const orc_geom* g, int32_t layer, uint8_t* const* dev, const uint8_t* host,
                        const int64_t* h, const int64_t* d, int64_t n);
int64_t orc_round_trip_check(const orc_geom* g, uint8_t* const* dev, const int64_t* a, const int64_t* c, int64_t n);
int orc_host_offsets(const orc_geom* g, int b, int32_t layer, const int64_t* h, int64_t n, int64_t* out);
int orc_h2h_dump(const orc_geom* pf, const orc_geom* sh, const uint8_t* host, uint8_t* store,
                 const int64_t* src_pages, const int64_t* dst_shards, int64_t n);
int orc_h2h_load(const orc_geom* pf, const orc_geom* sh, uint8_t* host, const uint8_t* store,
                 const int64_t* src_shards, const int64_t* dst_pages, int64_t n);
int64_t orc_layer_packed_bytes(const orc_geom* g, int64_t n);
int orc_layer_pack(const orc_geom* g, int32_t layer, uint8_t* const* dev, const int64_t* d, int64_t n, uint8_t* out);
int orc_layer_unpack(const orc_geom* g, int32_t layer, uint8_t* const* dev, const int64_t* d, int64_t n,
                     const uint8_t* in);

#endif
