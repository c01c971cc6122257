"""Oracle for the HiCache host<->device KV page transfer -- TEST INFRASTRUCTURE.

Thin numpy/ctypes wrapper around ``hc_oracle.c``, the plain C reference of the
indexed page copy.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product package
never imports it, and it imports nothing from the product package.

What it computes, and the passages it follows, is documented at the top of
``hc_oracle.c``: write-back of all layers (the staged write-back CPU mock of
the hybrid-pool write-back page, key source excerpts), per-layer load-back
(the loader-thread page, Motivation), the page_first_kv_split shard layout
with zero padding to the alignment (the CacheStore H2H page, section
"page_first_kv_split support"), a round-trip row comparison, and the per-layer
exchange of a rank-sharded host tier (the rank-sharded tier page, Modifications:
the owner packs a loaded layer's rows into staging, the other ranks unpack them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hc_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")

TOKEN_ROWS = 0
PAGE_BLOCKS = 1
PAGE_FIRST = 0
KV_SPLIT_SHARD = 1
PAGE_FIRST_TOKEN_MAJOR = 2
MAX_SUB = 4


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle into a shared library with gcc (plain -O2)."""
    cmd = ["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-I", _HERE, "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


class _Geom(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("nsub", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("host_pages", ctypes.c_int64),
        ("device_slots", ctypes.c_int64),
        ("align", ctypes.c_int64),
        ("gran", ctypes.c_int32 * MAX_SUB),
        ("bytes", ctypes.c_int64 * MAX_SUB),
    ]


_P64 = ctypes.POINTER(ctypes.c_int64)
_PU8 = ctypes.POINTER(ctypes.c_uint8)


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load an oracle library; the default one is compiled first when missing or stale."""
    if path == _LIB and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(_SRC, path)
    lib = ctypes.CDLL(path)
    G = ctypes.POINTER(_Geom)
    sig = {
        "orc_sub_page_bytes": (ctypes.c_int64, [G, ctypes.c_int]),
        "orc_page_payload_bytes": (ctypes.c_int64, [G]),
        "orc_shard_bytes": (ctypes.c_int64, [G]),
        "orc_host_pool_bytes": (ctypes.c_int64, [G]),
        "orc_host_offset": (ctypes.c_int64, [G, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
        "orc_device_offset": (ctypes.c_int64, [G, ctypes.c_int, ctypes.c_int64]),
        "orc_check_geom": (ctypes.c_int, [G]),
        "orc_check_indices": (ctypes.c_int, [G, _P64, _P64, ctypes.c_int64]),
        "orc_write_back": (ctypes.c_int, [G, ctypes.POINTER(_PU8), _PU8, _P64, _P64, ctypes.c_int64]),
        "orc_load_back_layer": (ctypes.c_int, [G, ctypes.c_int32, ctypes.POINTER(_PU8), _PU8, _P64, _P64, ctypes.c_int64]),
        "orc_round_trip_check": (ctypes.c_int64, [G, ctypes.POINTER(_PU8), _P64, _P64, ctypes.c_int64]),
        "orc_host_offsets": (ctypes.c_int, [G, ctypes.c_int, ctypes.c_int32, _P64, ctypes.c_int64, _P64]),
        "orc_h2h_dump": (ctypes.c_int, [G, G, _PU8, _PU8, _P64, _P64, ctypes.c_int64]),
        "orc_h2h_load": (ctypes.c_int, [G, G, _PU8, _PU8, _P64, _P64, ctypes.c_int64]),
        "orc_layer_packed_bytes": (ctypes.c_int64, [G, ctypes.c_int64]),
        "orc_layer_pack": (ctypes.c_int, [G, ctypes.c_int32, ctypes.POINTER(_PU8), _P64, ctypes.c_int64, _PU8]),
        "orc_layer_unpack": (ctypes.c_int, [G, ctypes.c_int32, ctypes.POINTER(_PU8), _P64, ctypes.c_int64, _PU8]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib_cache: dict[str, ctypes.CDLL] = {}
# HC_ORACLE_LIB lets a test run the pins against another build of the source.
_active = [os.environ.get("HC_ORACLE_LIB", _LIB)]


def lib(path: str | None = None) -> ctypes.CDLL:
    """The active oracle library (the built one unless ``use_library`` swapped it)."""
    path = path or _active[0]
    if path not in _lib_cache:
        _lib_cache[path] = load(path)
    return _lib_cache[path]


class use_library:
    """Context manager that routes every oracle call to another build of the
    oracle source (the tests use it to run the pins against planted mistakes)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        self.prev = _active[0]
        _active[0] = self.path
        return self

    def __exit__(self, *exc):
        _active[0] = self.prev
        return False


@dataclass
class Geometry:
    """Pool geometry: L layers, P tokens per page, sub-buffers (granularity, bytes)."""

    layers: int
    page_size: int
    subs: list  # [(TOKEN_ROWS | PAGE_BLOCKS, bytes per row or block)]
    host_pages: int
    device_slots: int
    layout: int = PAGE_FIRST
    align: int = 4096

    def c(self) -> _Geom:
        g = _Geom()
        g.layers, g.page_size, g.nsub, g.layout = self.layers, self.page_size, len(self.subs), self.layout
        g.host_pages, g.device_slots, g.align = self.host_pages, self.device_slots, self.align
        for b, (gran, nbytes) in enumerate(self.subs):
            g.gran[b] = gran
            g.bytes[b] = nbytes
        return g

    def device_units(self, b: int) -> int:
        """Rows (TOKEN) or blocks (PAGE) per device layer of sub-buffer b."""
        gran, _ = self.subs[b]
        return self.device_slots // self.page_size if gran == PAGE_BLOCKS else self.device_slots


def _i64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a


def _pi64(a: np.ndarray):
    return a.ctypes.data_as(_P64)


def _layer_table(g: Geometry, dev):
    """dev[b][l] -> flat C array of uint8 pointers, index b * L + l."""
    L = g.layers
    ptrs = (_PU8 * (len(g.subs) * L))()
    for b in range(len(g.subs)):
        for l in range(L):
            arr = dev[b][l]
            assert arr.dtype == np.uint8 and arr.flags.c_contiguous
            assert arr.nbytes >= g.device_units(b) * g.subs[b][1]
            ptrs[b * L + l] = arr.ctypes.data_as(_PU8)
    return ptrs


def sub_page_bytes(g: Geometry, b: int) -> int:
    return lib().orc_sub_page_bytes(ctypes.byref(g.c()), b)


def page_payload_bytes(g: Geometry) -> int:
    return lib().orc_page_payload_bytes(ctypes.byref(g.c()))


def shard_bytes(g: Geometry) -> int:
    return lib().orc_shard_bytes(ctypes.byref(g.c()))


def host_pool_bytes(g: Geometry) -> int:
    return lib().orc_host_pool_bytes(ctypes.byref(g.c()))


def host_offset(g: Geometry, b: int, page: int, layer: int, row: int) -> int:
    return lib().orc_host_offset(ctypes.byref(g.c()), b, page, layer, row)


def device_offset(g: Geometry, b: int, slot: int) -> int:
    return lib().orc_device_offset(ctypes.byref(g.c()), b, slot)


def host_offsets(g: Geometry, b: int, layer: int, h) -> np.ndarray:
    """Host byte offsets of the rows named by h (sub-buffer b, one layer)."""
    h = _i64(h)
    out = np.empty(h.size, dtype=np.int64)
    if lib().orc_host_offsets(ctypes.byref(g.c()), b, layer, _pi64(h), h.size, _pi64(out)) != 0:
        raise ValueError("oracle host_offsets rejected its arguments")
    return out


def check_geom(g: Geometry) -> bool:
    """Whether the oracle accepts the geometry (positive sizes, known layout and granularity, at
    most MAX_SUB sub-buffers, a positive shard alignment, whole device pages with page blocks)."""
    return lib().orc_check_geom(ctypes.byref(g.c())) == 0


def check_indices(g: Geometry, d, h) -> bool:
    d, h = _i64(d), _i64(h)
    if d.shape != h.shape:
        return False
    return lib().orc_check_indices(ctypes.byref(g.c()), _pi64(d), _pi64(h), d.size) == 0


def write_back(g: Geometry, dev, host: np.ndarray, d, h) -> None:
    """Write back all layers: host <- device rows named by (d, h).  In place on ``host``."""
    d, h = _i64(d), _i64(h)
    assert d.shape == h.shape
    assert host.dtype == np.uint8 and host.flags.c_contiguous and host.nbytes >= host_pool_bytes(g)
    rc = lib().orc_write_back(ctypes.byref(g.c()), _layer_table(g, dev), host.ctypes.data_as(_PU8),
                              _pi64(d), _pi64(h), d.size)
    if rc != 0:
        raise ValueError("oracle write_back rejected its arguments")


def load_back_layer(g: Geometry, layer: int, dev, host: np.ndarray, h, d) -> None:
    """Load back one layer: device rows named by d <- host rows named by h.  In place on ``dev``."""
    d, h = _i64(d), _i64(h)
    assert d.shape == h.shape
    assert host.dtype == np.uint8 and host.flags.c_contiguous and host.nbytes >= host_pool_bytes(g)
    rc = lib().orc_load_back_layer(ctypes.byref(g.c()), layer, _layer_table(g, dev),
                                   host.ctypes.data_as(_PU8), _pi64(h), _pi64(d), d.size)
    if rc != 0:
        raise ValueError("oracle load_back_layer rejected its arguments")


def round_trip_check(g: Geometry, dev, a, c) -> int:
    """Count (token, sub-buffer, layer) units whose rows at slots a[i] and c[i] differ."""
    a, c = _i64(a), _i64(c)
    assert a.shape == c.shape
    r = lib().orc_round_trip_check(ctypes.byref(g.c()), _layer_table(g, dev), _pi64(a), _pi64(c), a.size)
    if r < 0:
        raise ValueError("oracle round_trip_check rejected its arguments")
    return int(r)


def h2h_dump(pf: Geometry, sh: Geometry, host: np.ndarray, store: np.ndarray, src_pages, dst_shards) -> None:
    """Store shards dst_shards[i] <- host pages src_pages[i] (row by row), pads zeroed.  In place on ``store``."""
    a, b = _i64(src_pages), _i64(dst_shards)
    assert a.shape == b.shape and host.nbytes >= host_pool_bytes(pf) and store.nbytes >= host_pool_bytes(sh)
    rc = lib().orc_h2h_dump(ctypes.byref(pf.c()), ctypes.byref(sh.c()), host.ctypes.data_as(_PU8),
                            store.ctypes.data_as(_PU8), _pi64(a), _pi64(b), a.size)
    if rc != 0:
        raise ValueError("oracle h2h_dump rejected its arguments")


def h2h_load(pf: Geometry, sh: Geometry, host: np.ndarray, store: np.ndarray, src_shards, dst_pages) -> None:
    """Host pages dst_pages[i] <- store shards src_shards[i] (row by row).  In place on ``host``."""
    a, b = _i64(src_shards), _i64(dst_pages)
    assert a.shape == b.shape and host.nbytes >= host_pool_bytes(pf) and store.nbytes >= host_pool_bytes(sh)
    rc = lib().orc_h2h_load(ctypes.byref(pf.c()), ctypes.byref(sh.c()), host.ctypes.data_as(_PU8),
                            store.ctypes.data_as(_PU8), _pi64(a), _pi64(b), a.size)
    if rc != 0:
        raise ValueError("oracle h2h_load rejected its arguments")


def layer_packed_bytes(g: Geometry, n: int) -> int:
    """Bytes of one layer's exchange staging for n list entries."""
    r = lib().orc_layer_packed_bytes(ctypes.byref(g.c()), n)
    if r < 0:
        raise ValueError("oracle layer_packed_bytes rejected its arguments")
    return int(r)


def layer_pack(g: Geometry, layer: int, dev, d) -> np.ndarray:
    """Owner side of the layer exchange: the staging bytes of layer `layer` at slots d."""
    d = _i64(d)
    size = lib().orc_layer_packed_bytes(ctypes.byref(g.c()), d.size)  # -1: the call below rejects the list
    out = np.zeros(max(int(size), 1), dtype=np.uint8)
    rc = lib().orc_layer_pack(ctypes.byref(g.c()), layer, _layer_table(g, dev), _pi64(d), d.size,
                              out.ctypes.data_as(_PU8))
    if rc != 0:
        raise ValueError("oracle layer_pack rejected its arguments")
    return out[:size]


def layer_unpack(g: Geometry, layer: int, dev, d, packed: np.ndarray) -> None:
    """Receiving side of the layer exchange: rows of layer `layer` at slots d <- packed.  In place on ``dev``."""
    d = _i64(d)
    assert packed.dtype == np.uint8 and packed.flags.c_contiguous
    assert packed.nbytes >= lib().orc_layer_packed_bytes(ctypes.byref(g.c()), d.size)
    rc = lib().orc_layer_unpack(ctypes.byref(g.c()), layer, _layer_table(g, dev), _pi64(d), d.size,
                                packed.ctypes.data_as(_PU8))
    if rc != 0:
        raise ValueError("oracle layer_unpack rejected its arguments")
