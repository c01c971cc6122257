"""Host-to-host shard copies (CPU workers) against the oracle, queue capacity rules,
argument errors, and the cache-identity fingerprint."""
import ctypes

import numpy as np
import pytest

from host_device_page_amd import binding as B
from oracle import oracle as O

T, BL = O.TOKEN_ROWS, O.PAGE_BLOCKS


def pools(subs, L, P, H, S, shards, align):
    pf = O.Geometry(L, P, subs, H, S, O.PAGE_FIRST)
    sh = O.Geometry(L, P, subs, shards, S, O.KV_SPLIT_SHARD, align=align)
    d_pf, _k1 = B.make_desc(layers=L, page_size=P, subs=[(g, e, [16] * L) for g, e in subs], device_slots=S,
                            host_pages=H, layout=B.HC_LAYOUT_PAGE_FIRST)
    d_sh, _k2 = B.make_desc(layers=L, page_size=P, subs=[(g, e, [16] * L) for g, e in subs], device_slots=S,
                            host_pages=shards, layout=B.HC_LAYOUT_KV_SPLIT_SHARD, shard_align=align)
    return pf, sh, d_pf, d_sh, (_k1, _k2)


CASES = [
    ([(T, 2048), (T, 2048)], 3, 16, 24, 64, 20, 4096),     # K | V, no pad
    ([(T, 1024), (T, 128)], 3, 16, 24, 64, 20, 4096),      # K | V | 2048-byte pad
    ([(T, 1152), (BL, 8448)], 2, 64, 10, 128, 8, 4096),    # latent rows | indexer blocks | pad
    ([(T, 48)], 1, 1, 64, 64, 64, 256),                    # one-row pages
]


@pytest.mark.parametrize("workers", [0, 1, 4, 8])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_dump_and_load_match_oracle(ci, workers):
    subs, L, P, H, S, NS, align = CASES[ci]
    pf, sh, d_pf, d_sh, _keep = pools(subs, L, P, H, S, NS, align)
    rng = np.random.default_rng(ci * 10 + workers)
    host = rng.integers(0, 256, O.host_pool_bytes(pf), dtype=np.uint8)
    store = rng.integers(0, 256, O.host_pool_bytes(sh), dtype=np.uint8)
    n = min(H, NS) - 2
    src = rng.choice(H, size=n, replace=False)
    dst = rng.choice(NS, size=n, replace=False)
    stride = B.staging_page_bytes(d_sh)
    sizes = [O.sub_page_bytes(pf, b) for b in range(len(subs))]
    base = host.ctypes.data
    pages = [[base + B.host_offset(d_pf, b, int(p), 0, 0) for b in range(len(subs))] for p in src]
    shards = [store.ctypes.data + int(q) * stride for q in dst]
    want = store.copy()
    O.h2h_dump(pf, sh, host, want, src, dst)
    eng = B.H2H(workers=workers, queue_depth=4096)
    eng.wait(eng.submit(B.HC_H2H_DUMP, sizes, pages, shards, stride))
    assert np.array_equal(store, want), "dump differs from the oracle"
    assert eng.outstanding() == (0, 0)
    # load into other pages
    back = rng.integers(0, 256, host.size, dtype=np.uint8)
    dst_pages = rng.choice(H, size=n, replace=False)
    want_back = back.copy()
    O.h2h_load(pf, sh, want_back, store, dst, dst_pages)
    pages2 = [[back.ctypes.data + B.host_offset(d_pf, b, int(p), 0, 0) for b in range(len(subs))] for p in dst_pages]
    eng.wait(eng.submit(B.HC_H2H_LOAD, sizes, pages2, shards, stride))
    assert np.array_equal(back, want_back), "load differs from the oracle"
    eng.close()


def test_capacity_is_reserved_for_the_whole_request():
    eng = B.H2H(workers=0, queue_depth=8)  # manual progress: jobs run at wait
    buf = np.zeros(64 * 16, dtype=np.uint8)
    a = buf.ctypes.data
    r1 = eng.submit(B.HC_H2H_DUMP, [16], [[a + 16 * i] for i in range(5)], [a + 512 + 16 * i for i in range(5)], 16)
    assert eng.outstanding() == (5, 0)
    with pytest.raises(B.HcError) as e:
        eng.submit(B.HC_H2H_DUMP, [16], [[a] for _ in range(4)], [a + 900 + 16 * i for i in range(4)], 16)
    assert e.value.code == B.HC_ERR_BUSY
    assert eng.outstanding() == (5, 0), "a refused request must not hold capacity"
    r2 = eng.submit(B.HC_H2H_LOAD, [16], [[a + 16 * i] for i in range(8)], [a + 512 + 16 * i for i in range(8)], 16)
    assert eng.outstanding() == (5, 8), "load and dump are counted apart"
    eng.wait(r1)
    assert eng.outstanding() == (0, 8)
    eng.wait(r2)
    assert eng.outstanding() == (0, 0)
    eng.close()


def test_refused_requests():
    eng = B.H2H(workers=2, queue_depth=16)
    buf = np.zeros(1024, dtype=np.uint8)
    a = buf.ctypes.data
    with pytest.raises(B.HcError) as e:
        eng.submit(B.HC_H2H_DUMP, [64, 64], [[a, 0]], [a + 512], 256)  # null tensor page
    assert e.value.code == B.HC_ERR_INVALID
    with pytest.raises(B.HcError):
        eng.submit(B.HC_H2H_DUMP, [64, 64], [[a, a]], [0], 256)  # null shard
    with pytest.raises(B.HcError):
        eng.submit(B.HC_H2H_DUMP, [200, 100], [[a, a]], [a + 512], 256)  # pages do not fit the shard
    with pytest.raises(B.HcError):
        eng.submit(7, [16], [[a]], [a + 512], 16)
    with pytest.raises(B.HcError) as e:  # more shards than the queue holds: never admissible, not "busy"
        eng.submit(B.HC_H2H_DUMP, [16], [[a] for _ in range(17)], [a + 512 + 16 * i for i in range(17)], 16)
    assert e.value.code == B.HC_ERR_INVALID and "queue depth" in str(e.value)
    assert eng.outstanding() == (0, 0)
    out = ctypes.c_void_p()
    assert B.lib.hc_h2h_create(-1, 4, ctypes.byref(out)) == B.HC_ERR_INVALID
    assert B.lib.hc_h2h_create(2, 0, ctypes.byref(out)) == B.HC_ERR_INVALID
    eng.close()


def fnv1a64(text: str) -> int:
    h = 0xcbf29ce484222325
    for c in text.encode():
        h = ((h ^ c) * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a_reference_values():
    # values of the published FNV-1a 64-bit test suite
    assert fnv1a64("") == 0xcbf29ce484222325
    assert fnv1a64("a") == 0xaf63dc4c8601ec8c
    assert fnv1a64("foobar") == 0x85944171f73967e8


def test_cache_fingerprint():
    def desc(**kw):
        base = dict(layers=61, page_size=64, subs=[(0, 1152, [16] * 61)], device_slots=524288, host_pages=16384,
                    layout=B.HC_LAYOUT_PAGE_FIRST)
        base.update(kw)
        return B.make_desc(**base)

    d, _k = desc()
    fp = B.cache_fingerprint(d, "deepseek-v3", 8)
    assert fp == fnv1a64("hicache-layout-v1;model=deepseek-v3;layout=page_first;layers=61;page_size=64;tp=8;"
                         "tensors=r:1152;align=0")
    assert fp == B.cache_fingerprint(d, "deepseek-v3", 8)
    others = [
        B.cache_fingerprint(d, "deepseek-v3.1", 8),
        B.cache_fingerprint(d, "deepseek-v3", 4),
        B.cache_fingerprint(desc(layout=B.HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR)[0], "deepseek-v3", 8),
        B.cache_fingerprint(desc(page_size=32)[0], "deepseek-v3", 8),
        B.cache_fingerprint(desc(subs=[(0, 1152, [16] * 61), (1, 8448, [16] * 61)])[0], "deepseek-v3", 8),
        B.cache_fingerprint(desc(layout=B.HC_LAYOUT_KV_SPLIT_SHARD, shard_align=4096)[0], "deepseek-v3", 8),
    ]
    assert len(set(others + [fp])) == len(others) + 1, "a layout change kept the fingerprint"
    # host page count and device slots are capacity, not layout
    assert B.cache_fingerprint(desc(host_pages=100)[0], "deepseek-v3", 8) == fp


def test_destroy_refuses_while_a_request_is_not_released():
    eng = B.H2H(workers=2, queue_depth=16)
    buf = np.zeros(4096, dtype=np.uint8)
    a = buf.ctypes.data
    req = eng.submit(B.HC_H2H_DUMP, [64], [[a + 64 * i] for i in range(4)], [a + 2048 + 64 * i for i in range(4)], 64)
    assert B.lib.hc_h2h_destroy(eng.handle) == B.HC_ERR_INVALID
    assert "not released" in B.lib.hc_last_error().decode()
    eng.close()  # the binding waits for and releases the request first
    assert not eng.handle.value
    assert np.array_equal(buf[2048:2048 + 256], buf[0:256])
    del req
