"""The C ABI without a GPU: exported symbols, descriptor checks, layout arithmetic.

Nothing here launches work: the calls used run on the CPU only (descriptor and
layout queries, argument errors returned before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from host_device_page_amd import binding as B
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hc_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(B.lib, n), f"{n} declared in hc.h but not exported by libhc.so"
    assert set(names) == set(B._SIGS), "binding and header disagree"
    assert B.lib.hc_version() >= 1


def desc(**kw):
    base = dict(layers=4, page_size=16, subs=[(B.HC_TOKEN_ROWS, 1024, [0x10000 * (i + 1) for i in range(4)])] * 2,
                device_slots=4096, host_pages=256, host_ptr=0x7f0000000000, host_bytes=1 << 40)
    base.update(kw)
    return B.make_desc(**base)


def status(d):
    return B.lib.hc_desc_check(ctypes.byref(d))


def test_desc_check_accepts_valid():
    d, _k = desc()
    assert status(d) == B.HC_OK, B.lib.hc_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(layers=0), B.HC_ERR_INVALID, "num_layers"),
    (dict(page_size=0), B.HC_ERR_INVALID, "page_size"),
    (dict(device_slots=0), B.HC_ERR_INVALID, "device_slots"),
    (dict(subs=[(B.HC_TOKEN_ROWS, 1000, [0x10000] * 4)]), B.HC_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(subs=[(B.HC_TOKEN_ROWS, 131072, [0x10000] * 4)]), B.HC_ERR_UNSUPPORTED, "HC_MAX_ELEM_BYTES"),
    (dict(subs=[(7, 1024, [0x10000] * 4)]), B.HC_ERR_INVALID, "granularity"),
    (dict(subs=[(B.HC_TOKEN_ROWS, 1024, [0x10000, 0, 0x10000, 0x10000])]), B.HC_ERR_INVALID, "null device pointer"),
    (dict(subs=[(B.HC_TOKEN_ROWS, 1024, [0x10008] * 4)]), B.HC_ERR_UNSUPPORTED, "16-byte aligned"),
    (dict(subs=[(B.HC_PAGE_BLOCKS, 1024, [0x10000] * 4)], device_slots=4097), B.HC_ERR_INVALID, "multiple of page_size"),
    (dict(layout=B.HC_LAYOUT_KV_SPLIT_SHARD, shard_align=3000), B.HC_ERR_INVALID, "power of two"),
    (dict(layout=5), B.HC_ERR_INVALID, "layout"),
    (dict(host_ptr=0), B.HC_ERR_INVALID, "host_base"),
    (dict(host_ptr=0x7f0000000008), B.HC_ERR_UNSUPPORTED, "host_base"),
    (dict(host_bytes=100), B.HC_ERR_INVALID, "host_bytes"),
    (dict(write_back_mode=B.HC_MODE_STAGED), B.HC_ERR_INVALID, "staging"),
    (dict(write_back_mode=B.HC_MODE_STAGED, staging_ptr=0x20000, staging_bytes=1000), B.HC_ERR_INVALID, "staging"),
    (dict(load_back_mode=B.HC_MODE_STAGED), B.HC_ERR_UNSUPPORTED, "staged load-back"),
    (dict(write_back_mode=9), B.HC_ERR_INVALID, "mode"),
    (dict(flags=64), B.HC_ERR_INVALID, "flags"),
    (dict(device_slots=1 << 60), B.HC_ERR_INVALID, "device layer size overflows"),
    (dict(max_ctas=-1), B.HC_ERR_INVALID, "max_ctas"),
    (dict(max_ctas=65537), B.HC_ERR_INVALID, "max_ctas"),
    (dict(host_pages=-1), B.HC_ERR_INVALID, "host_pages"),
    # a device-only pool (host_pages = 0) takes no host memory and no write-back staging
    (dict(host_pages=0), B.HC_ERR_INVALID, "takes no host_base"),
    (dict(host_pages=0, host_ptr=0, write_back_mode=B.HC_MODE_STAGED), B.HC_ERR_INVALID, "no write-back"),
    (dict(host_pages=0, host_ptr=0, staging_ptr=0x20000, staging_bytes=1 << 30), B.HC_ERR_INVALID, "no staging"),
])
def test_desc_check_rejects(kw, code, text):
    d, _k = desc(**kw)
    assert status(d) == code
    assert text in B.lib.hc_last_error().decode()


def test_device_only_descriptor():
    """host_pages = 0: no host pool at all (host_base NULL, 0 host bytes, no page offsets)."""
    d, _k = desc(host_pages=0, host_ptr=0, host_bytes=0)
    assert status(d) == B.HC_OK, B.lib.hc_last_error()
    out = ctypes.c_int64(-1)
    assert B.lib.hc_host_pool_bytes(ctypes.byref(d), ctypes.byref(out)) == B.HC_OK and out.value == 0
    assert B.lib.hc_host_offset(ctypes.byref(d), 0, 0, 0, 0, ctypes.byref(out)) == B.HC_ERR_INVALID


def test_null_arguments_without_gpu():
    assert B.lib.hc_desc_check(None) == B.HC_ERR_INVALID
    assert B.lib.hc_pool_destroy(None) == B.HC_OK
    assert B.lib.hc_write_back_all_layers(None, None, None, 0, None) == B.HC_ERR_INVALID
    assert B.lib.hc_write_back_all_layers_noalloc(None, None, None, 0, None) == B.HC_ERR_INVALID
    # a null pool with a null event: reported, nothing recorded
    assert B.lib.hc_load_back_layer(None, 0, None, None, 0, None) == B.HC_ERR_INVALID
    assert B.lib.hc_round_trip_check(None, None, None, 0, None) == B.HC_ERR_INVALID
    assert B.lib.hc_pool_sync(None) == B.HC_ERR_INVALID
    out = ctypes.c_void_p()
    assert B.lib.hc_host_alloc(0, 0, ctypes.byref(out)) == B.HC_ERR_INVALID
    assert B.lib.hc_pool_create(None, ctypes.byref(out)) == B.HC_ERR_INVALID
    evs = (ctypes.c_void_p * 1)()
    assert B.lib.hc_load_back_graph_create(None, None, None, 0, evs, ctypes.byref(out)) == B.HC_ERR_INVALID
    assert out.value is None
    assert B.lib.hc_load_back_graph_create(None, None, None, 0, evs, None) == B.HC_ERR_INVALID
    assert B.lib.hc_load_back_graph_launch(None) == B.HC_ERR_INVALID
    assert B.lib.hc_pool_get_stats(None, ctypes.byref(B.hc_pool_stats())) == B.HC_ERR_INVALID
    assert B.lib.hc_load_back_graph_destroy(None) == B.HC_OK
    n = ctypes.c_int64()
    assert B.lib.hc_layer_pack_bytes(None, 64, ctypes.byref(n)) == B.HC_ERR_INVALID
    assert B.lib.hc_layer_pack(None, 0, None, 0, None, 0, None) == B.HC_ERR_INVALID
    assert B.lib.hc_layer_unpack(None, 0, None, 0, None, 0, None) == B.HC_ERR_INVALID


GEOMS = [
    dict(layers=4, page_size=16, subs=[(0, 1024), (0, 1024)], host_pages=256, device_slots=4096, layout=0),
    dict(layers=48, page_size=32, subs=[(0, 2048), (0, 2048)], host_pages=4096, device_slots=262144, layout=1),
    dict(layers=3, page_size=16, subs=[(0, 1024), (0, 128)], host_pages=40, device_slots=4096, layout=1),
    dict(layers=78, page_size=64, subs=[(0, 1152), (1, 8448)], host_pages=2048, device_slots=524288, layout=0),
    dict(layers=78, page_size=64, subs=[(0, 1152), (1, 8448)], host_pages=2048, device_slots=524288, layout=1),
    dict(layers=1, page_size=16, subs=[(0, 48), (0, 16), (1, 32), (0, 64)], host_pages=64, device_slots=2048, layout=0),
    dict(layers=61, page_size=64, subs=[(0, 1152)], host_pages=16384, device_slots=524288, layout=0),
    dict(layers=5, page_size=7, subs=[(1, 16), (0, 32)], host_pages=9, device_slots=70, layout=1),
    dict(layers=32, page_size=64, subs=[(0, 2048), (0, 2048)], host_pages=8192, device_slots=262144, layout=2),
    dict(layers=78, page_size=64, subs=[(0, 1152), (1, 8448)], host_pages=2048, device_slots=524288, layout=2),
    dict(layers=5, page_size=7, subs=[(1, 16), (0, 32), (0, 48)], host_pages=9, device_slots=70, layout=2),
]


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_layout_arithmetic_matches_oracle(gi):
    g = GEOMS[gi]
    og = O.Geometry(g["layers"], g["page_size"], g["subs"], g["host_pages"], g["device_slots"], g["layout"], 4096)
    d, _k = B.make_desc(layers=g["layers"], page_size=g["page_size"],
                        subs=[(gr, e, [0x10000] * g["layers"]) for gr, e in g["subs"]],
                        device_slots=g["device_slots"], host_pages=g["host_pages"], layout=g["layout"],
                        shard_align=4096)
    assert B.host_pool_bytes(d) == O.host_pool_bytes(og)
    want_img = O.shard_bytes(og) if g["layout"] == 1 else O.page_payload_bytes(og)
    assert B.staging_page_bytes(d) == want_img
    rng = np.random.default_rng(gi)
    for _ in range(300):
        b = int(rng.integers(0, len(g["subs"])))
        p = int(rng.integers(0, g["host_pages"]))
        l = int(rng.integers(0, g["layers"]))
        r = int(rng.integers(0, g["page_size"]))
        assert B.host_offset(d, b, p, l, r) == O.host_offset(og, b, p, l, r), (b, p, l, r)
    # corners
    for b in range(len(g["subs"])):
        for p in (0, g["host_pages"] - 1):
            for l in (0, g["layers"] - 1):
                for r in (0, g["page_size"] - 1):
                    assert B.host_offset(d, b, p, l, r) == O.host_offset(og, b, p, l, r)
    out = ctypes.c_int64()
    assert B.lib.hc_host_offset(ctypes.byref(d), 0, g["host_pages"], 0, 0, ctypes.byref(out)) == B.HC_ERR_INVALID
    assert B.lib.hc_host_offset(ctypes.byref(d), 0, 0, g["layers"], 0, ctypes.byref(out)) == B.HC_ERR_INVALID


def test_header_constants_match_the_binding():
    """Every numeric #define of hc.h that the binding also names has the same value there."""
    text = open(HEADER).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(HC_[A-Z0-9_]+)\s+(\d+)\b", text)}
    assert {"HC_MAX_SUBBUFS", "HC_DUPLEX_LOAD_BACK_CTAS", "HC_NOALLOC_MAX_TOKENS"} <= set(defs)
    # enumerators too (modes, layouts, flags, status codes)
    body = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for m in re.finditer(r"\b(HC_[A-Z0-9_]+)\s*=\s*(-?\d+)", body):
        defs[m.group(1)] = int(m.group(2))
    assert {"HC_FLAG_PROFILE", "HC_MODE_STAGED", "HC_ERR_DEVICE"} <= set(defs)
    shared = [k for k in defs if hasattr(B, k)]
    assert {"HC_DUPLEX_LOAD_BACK_CTAS", "HC_FLAG_PROFILE", "HC_LAYOUT_KV_SPLIT_SHARD", "HC_ERR_DEVICE"} <= set(shared)
    for k in shared:
        assert getattr(B, k) == defs[k], k
