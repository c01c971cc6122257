"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
import os
import subprocess
import sys
import tempfile

import pytest

import pins
from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes, planted in a copy of the oracle source.  Each must make at
# least one pin fail (or crash the pin run): a dropped term, a wrong index, a
# transposed operand, a missing rounding step, a wrong fill value.
MUTANTS = [
    ("layer and row transposed in the host offset",
     "inner = ((int64_t)l * g->page_size + r) * g->bytes[b];",
     "inner = ((int64_t)r * g->layers + l) * g->bytes[b];"),
    ("token-major rows laid out layer-major",
     "inner = ((int64_t)r * g->layers + l) * g->bytes[b];",
     "inner = ((int64_t)l * g->page_size + r) * g->bytes[b];"),
    ("store shard pad left as it was",
     "memset(store + dst_shards[i] * stride + payload, 0, (size_t)(stride - payload));", ";"),
    ("store load reads the destination page's shard",
     "store + orc_host_offset(sh, b, src_shards[i], l, r),", "store + orc_host_offset(sh, b, dst_pages[i] % sh->host_pages, l, r),"),
    ("write-back carries state between calls (pad written only on the first call)",
     "  if (g->layout == ORC_KV_SPLIT_SHARD) {\n    int64_t payload = orc_page_payload_bytes(g);",
     "  static int calls = 0;\n  if (g->layout == ORC_KV_SPLIT_SHARD && calls++ == 0) {\n    int64_t payload = orc_page_payload_bytes(g);"),
    ("write-back drops the last token of a burst",
     "  for (int64_t i = 0; i < n; i++) {\n    int64_t page = h[i] / P;\n    int32_t row = (int32_t)(h[i] % P);\n    for (int b = 0; b < g->nsub; b++) {\n      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;\n      for (int l = 0; l < L; l++) {",
     "  for (int64_t i = 0; i + 1 < n; i++) {\n    int64_t page = h[i] / P;\n    int32_t row = (int32_t)(h[i] % P);\n    for (int b = 0; b < g->nsub; b++) {\n      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;\n      for (int l = 0; l < L; l++) {"),
    ("shard size not rounded up",
     "if (k * a < s) k = k + 1;", ";"),
    ("sub-buffer region ignores the page count",
     "region += g->host_pages * orc_sub_page_bytes(g, c);",
     "region += orc_sub_page_bytes(g, c);"),
    ("earlier sub-buffers dropped inside a shard",
     "for (int c = 0; c < b; c++) before += orc_sub_page_bytes(g, c);", ";"),
    ("page block indexed by token slot",
     "if (g->gran[b] == ORC_PAGE_BLOCKS) return (s / g->page_size) * g->bytes[b];",
     "if (g->gran[b] == ORC_PAGE_BLOCKS) return s * g->bytes[b];"),
    ("row off by one in write-back",
     "int32_t row = (int32_t)(h[i] % P);\n    for (int b = 0; b < g->nsub; b++) {\n      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;\n      for (int l = 0; l < L; l++) {",
     "int32_t row = (int32_t)((h[i] + 1) % P);\n    for (int b = 0; b < g->nsub; b++) {\n      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;\n      for (int l = 0; l < L; l++) {"),
    ("pad filled with a nonzero byte",
     "memset(host + page * stride + payload, 0,", "memset(host + page * stride + payload, 1,"),
    ("pad never written",
     "memset(host + page * stride + payload, 0, (size_t)(stride - payload));", ";"),
    ("load-back always writes layer 0",
     "uint8_t* dst = dev[b * L + layer] + orc_device_offset(g, b, d[i]);",
     "uint8_t* dst = dev[b * L + 0] + orc_device_offset(g, b, d[i]);"),
    ("load-back reads layer 0 of the host page",
     "const uint8_t* src = host + orc_host_offset(g, b, page, layer, row);",
     "const uint8_t* src = host + orc_host_offset(g, b, page, 0, row);"),
    ("misaligned device page accepted for page blocks",
     "if (first < 0 || first % g->page_size != 0) { rc = ORC_ERR_INVALID; break; }",
     "if (first < 0) { rc = ORC_ERR_INVALID; break; }"),
    ("round-trip check counts equal rows",
     "if (memcmp(x, y, (size_t)g->bytes[b]) != 0) bad++;",
     "if (memcmp(x, y, (size_t)g->bytes[b]) == 0) bad++;"),
    ("repeated host tokens accepted",
     "if (seen_d[d[i]] || seen_h[h[i]]) {", "if (seen_d[d[i]]) {"),
    ("device and host index swapped in write-back",
     "const uint8_t* src = dev[b * L + l] + orc_device_offset(g, b, d[i]);",
     "const uint8_t* src = dev[b * L + l] + orc_device_offset(g, b, h[i] % g->device_slots);"),
    ("exchange pack reads layer 0",
     "memcpy(at, dev[b * L + layer] + orc_device_offset(g, b, d[i]), (size_t)g->bytes[b]);",
     "memcpy(at, dev[b * L + 0] + orc_device_offset(g, b, d[i]), (size_t)g->bytes[b]);"),
    ("exchange unpack writes layer 0",
     "memcpy(dev[b * L + layer] + orc_device_offset(g, b, d[i]), at, (size_t)g->bytes[b]);",
     "memcpy(dev[b * L + 0] + orc_device_offset(g, b, d[i]), at, (size_t)g->bytes[b]);"),
    ("exchange pack takes a page block at every token",
     "  uint8_t* at = out;\n  for (int b = 0; b < g->nsub; b++) {\n    const int64_t step = g->gran[b] == ORC_PAGE_BLOCKS ? g->page_size : 1;",
     "  uint8_t* at = out;\n  for (int b = 0; b < g->nsub; b++) {\n    const int64_t step = 1;"),
    ("exchange unpack reads staging one row late",
     "const uint8_t* at = in;", "const uint8_t* at = in + g->bytes[0];"),
    ("exchange accepts a page that does not start at a multiple of P",
     "if (d[k] % P != 0) return ORC_ERR_INVALID;", ";"),
    ("exchange accepts repeated slots",
     "if (d[i] < 0 || d[i] >= g->device_slots || seen[d[i]]) { rc = ORC_ERR_INVALID; break; }",
     "if (d[i] < 0 || d[i] >= g->device_slots) { rc = ORC_ERR_INVALID; break; }"),
    ("exchange staging size counts page blocks per token",
     "total += (n / g->page_size) * g->bytes[b];", "total += n * g->bytes[b];"),
    ("batched host offsets swap page and row",
     "out[i] = orc_host_offset(g, b, h[i] / g->page_size, layer, (int32_t)(h[i] % g->page_size));",
     "out[i] = orc_host_offset(g, b, h[i] % g->page_size, layer, (int32_t)(h[i] / g->page_size));"),
    ("batched host offsets ignore the layer",
     "out[i] = orc_host_offset(g, b, h[i] / g->page_size, layer, (int32_t)(h[i] % g->page_size));",
     "out[i] = orc_host_offset(g, b, h[i] / g->page_size, 0, (int32_t)(h[i] % g->page_size));"),
    ("batched host offsets take the row of the next token",
     "out[i] = orc_host_offset(g, b, h[i] / g->page_size, layer, (int32_t)(h[i] % g->page_size));",
     "out[i] = orc_host_offset(g, b, h[i] / g->page_size, layer, (int32_t)((h[i] + 1) % g->page_size));"),
    ("batched host offsets accept the first token past the pool",
     "if (h[i] < 0 || h[i] >= g->host_pages * g->page_size) return ORC_ERR_INVALID;",
     "if (h[i] < 0 || h[i] > g->host_pages * g->page_size) return ORC_ERR_INVALID;"),
    ("batched host offsets accept a layer past the last",
     "b < 0 || b >= g->nsub || layer < 0 || layer >= g->layers) return ORC_ERR_INVALID;",
     "b < 0 || b >= g->nsub || layer < 0 || layer > g->layers) return ORC_ERR_INVALID;"),
    ("geometry without sub-buffers accepted",
     "g->nsub <= 0 || g->nsub > ORC_MAX_SUB)", "g->nsub > ORC_MAX_SUB)"),
    ("geometry with five sub-buffers accepted",
     "g->nsub <= 0 || g->nsub > ORC_MAX_SUB)", "g->nsub <= 0 || g->nsub > ORC_MAX_SUB + 1)"),
    ("shard alignment of 0 accepted",
     "if (g->layout == ORC_KV_SPLIT_SHARD && g->align <= 0) return ORC_ERR_INVALID;", ";"),
    ("page blocks over a partial device page accepted",
     "if (has_page_blocks(g) && g->device_slots % g->page_size != 0) return ORC_ERR_INVALID;", ";"),
    ("unknown granularity accepted",
     "if (g->gran[b] != ORC_TOKEN_ROWS && g->gran[b] != ORC_PAGE_BLOCKS) return ORC_ERR_INVALID;", ";"),
    ("load-back writes one slot past the listed one",
     "uint8_t* dst = dev[b * L + layer] + orc_device_offset(g, b, d[i]);",
     "uint8_t* dst = dev[b * L + layer] + orc_device_offset(g, b, (d[i] + 1) % g->device_slots);"),
    ("store dump copies only the first sub-buffer",
     "    for (int b = 0; b < pf->nsub; b++) {\n      int32_t rows = pf->gran[b] == ORC_PAGE_BLOCKS ? 1 : pf->page_size;\n"
     "      for (int32_t l = 0; l < pf->layers; l++)\n        for (int32_t r = 0; r < rows; r++)\n"
     "          memcpy(store + orc_host_offset(sh, b, dst_shards[i], l, r)",
     "    for (int b = 0; b < 1; b++) {\n      int32_t rows = pf->gran[b] == ORC_PAGE_BLOCKS ? 1 : pf->page_size;\n"
     "      for (int32_t l = 0; l < pf->layers; l++)\n        for (int32_t r = 0; r < rows; r++)\n"
     "          memcpy(store + orc_host_offset(sh, b, dst_shards[i], l, r)"),
    ("round-trip check skips page-block sub-buffers",
     "if (g->gran[b] == ORC_PAGE_BLOCKS && a[i] % P != 0) continue;",
     "if (g->gran[b] == ORC_PAGE_BLOCKS) continue;"),
    ("write-back writes into the next host page",
     "uint8_t* dst = host + orc_host_offset(g, b, page, l, row);",
     "uint8_t* dst = host + orc_host_offset(g, b, (page + 1) % g->host_pages, l, row);"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(desc, old, new):
    src = open(os.path.join(os.path.dirname(O.__file__), "hc_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {desc}"
    with tempfile.TemporaryDirectory() as tmp:
        msrc = os.path.join(tmp, "mutant.c")
        mlib = os.path.join(tmp, "libmutant.so")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new, 1))
        O.build(msrc, mlib)
        env = dict(os.environ, HC_ORACLE_LIB=mlib)
        r = subprocess.run([sys.executable, os.path.join(HERE, "pins.py")], env=env,
                           capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch: {desc}\n{r.stdout}"
