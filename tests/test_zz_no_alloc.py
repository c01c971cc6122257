"""The write-back that allocates nothing (hc_write_back_all_layers_noalloc) against the
ordinary write-back (hc_write_back_all_layers) and the oracle.

Two zero-copy pools share one device pool; each has its own pinned host pool.  The
ordinary write-back fills one host pool, the no-allocation write-back the other, for two
bursts in a row, the second smaller than the first (the library's scratch still holds
the first burst's list behind the second's).  After each burst both host pools must be
byte-identical to each other and to the oracle's.  Device memory must not change across
the no-allocation calls."""
import ctypes

import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, assert_bytes_equal, cuda_i64, say
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
PF, SH, TM = W.PAGE_FIRST, W.KV_SPLIT_SHARD, W.PAGE_FIRST_TOKEN_MAJOR
FILL = 0xA5
MAX = 262144  # HC_NOALLOC_MAX_TOKENS


def S(name, L, P, subs, slots, pages, layout=PF, align=4096):
    return W.PoolShape(name, L, P, tuple(subs), slots, pages, layout, align)


SHAPES = [
    W.SHAPES["tiny_mha_bf16"],
    S("na_shard_pad", 3, 16, [(T, 1024), (T, 128)], 4096, 40, SH),
    S("na_indexer", 3, 64, [(T, 1152), (BLK, 8448)], 8192, 32),
    S("na_token_major", 4, 16, [(T, 2048), (T, 512)], 8192, 64, TM),
]


def has_blocks(shape):
    return any(g == BLK for g, _ in shape.subs)


def burst(shape, pages, seed):
    """Host tokens and device slots.  Token-row pools: pages named in part, tokens of
    different pages interleaved (a page's tokens form several runs).  Page-block pools:
    whole pages in row order onto whole, page-aligned device pages."""
    rng = np.random.default_rng(seed)
    P = shape.page_size
    pg = rng.choice(shape.host_pages, size=pages, replace=False)
    if has_blocks(shape):
        h = W.whole_page_tokens(pg, P)
        d = W.page_aligned_slots(seed + 1, shape.device_slots, P, pages)
        return h, d
    toks = [p * P + np.sort(rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False)) for p in pg]
    h = np.concatenate(toks).astype(np.int64)
    h = h[rng.permutation(h.size)]
    d = rng.choice(shape.device_slots, size=h.size, replace=False).astype(np.int64)
    return h, d


class Pair:
    """Pool A (ordinary write-back, the Rig's host pool) and pool B (no-allocation
    write-back, its own host pool) over the same device buffers and copy stream."""

    def __init__(self, shape, seed):
        self.rig = Rig(shape, seed=seed, host_fill=FILL)
        L = shape.layers
        self.host_b = B.HostBuffer(self.rig.host_bytes)
        self.host_b.fill(FILL)
        self.pool_b = B.Pool(layers=L, page_size=shape.page_size, subs=list(shape.subs),
                             device_slots=shape.device_slots, host_pages=shape.host_pages,
                             device_layers=[[self.rig.dev[b][l] for l in range(L)] for b in range(len(shape.subs))],
                             host=self.host_b, stream=self.rig.stream, layout=shape.layout,
                             shard_align=shape.align, write_back_mode=B.HC_MODE_ZEROCOPY)
        self.lists = B.HostBuffer(8 * MAX)

    def close(self):
        self.pool_b.close()
        self.host_b.free()
        self.lists.free()
        self.rig.close()


def run_pair(pair, h, d, what):
    rig = pair.rig
    n = h.size
    dev0 = rig.dev_np()
    want = rig.host.np.copy()
    O.write_back(rig.geom, dev0, want, d, h)
    d_t = cuda_i64(d)
    torch.cuda.synchronize()
    rig.pool.write_back_all_layers(d_t, h)
    rig.pool.sync()
    pair.lists.np.view(np.int64)[:n] = h
    free0 = torch.cuda.mem_get_info()[0]
    pair.pool_b.write_back_all_layers_noalloc(d_t, pair.lists, n)
    pair.pool_b.sync()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, f"{what}: free device memory changed across the no-allocation call ({free0} -> {free1})"
    assert_bytes_equal(rig.host.np, want, f"{what}: ordinary write-back against the oracle")
    assert_bytes_equal(pair.host_b.np, rig.host.np, f"{what}: no-allocation write-back against the ordinary one")


@pytest.mark.gpu
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_no_alloc_write_back_equals_the_ordinary_one(shape):
    say(f"[noalloc] {shape.name}")
    pair = Pair(shape, seed=11)
    try:
        big = min(shape.host_pages, 24)
        h1, d1 = burst(shape, big, 100)
        h2, d2 = burst(shape, max(1, big // 3), 200)
        assert h2.size < h1.size
        run_pair(pair, h1, d1, f"{shape.name} first burst ({h1.size} tokens)")
        run_pair(pair, h2, d2, f"{shape.name} second, smaller burst ({h2.size} tokens)")
        st = pair.pool_b.stats()
        assert st["write_back_calls"] == 2 and st["write_back_tokens"] == h1.size + h2.size
    finally:
        pair.close()


@pytest.mark.gpu
def test_no_alloc_write_back_at_its_maximum_then_smaller():
    """n = HC_NOALLOC_MAX_TOKENS (every token of the pool), then a ragged smaller burst."""
    shape = S("na_max", 2, 64, [(T, 32), (T, 16)], MAX, MAX // 64)
    say(f"[noalloc] {shape.name}")
    pair = Pair(shape, seed=12)
    try:
        rng = np.random.default_rng(300)
        h1 = rng.permutation(MAX).astype(np.int64)
        d1 = rng.permutation(MAX).astype(np.int64)
        run_pair(pair, h1, d1, "maximum burst")
        h2, d2 = burst(shape, 37, 301)
        run_pair(pair, h2, d2, "smaller burst after the maximum")
    finally:
        pair.close()


@pytest.mark.gpu
def test_no_alloc_write_back_refusals():
    """Refused before anything is enqueued: n above the maximum, a host list in pageable
    memory, a staged pool; the host pool keeps its bytes."""
    shape = SHAPES[0]
    say("[noalloc] refusals")
    pair = Pair(shape, seed=13)
    staged = None
    try:
        rig = pair.rig
        h, d = burst(shape, 4, 400)
        n = h.size
        pair.lists.np.view(np.int64)[:n] = h
        d_t = cuda_i64(d)
        big_d = torch.zeros(MAX + 1, dtype=torch.int64, device="cuda")
        big_h = B.HostBuffer(8 * (MAX + 1))
        try:
            code = B.lib.hc_write_back_all_layers_noalloc(pair.pool_b.handle, ctypes.c_void_p(big_d.data_ptr()),
                                                          big_h.ptr, MAX + 1, None)
            assert code == B.HC_ERR_INVALID and b"above" in B.lib.hc_last_error()
        finally:
            big_h.free()
        pageable = np.ascontiguousarray(h)
        code = B.lib.hc_write_back_all_layers_noalloc(pair.pool_b.handle, ctypes.c_void_p(d_t.data_ptr()),
                                                      ctypes.c_void_p(pageable.ctypes.data), n, None)
        assert code == B.HC_ERR_INVALID and b"pinned" in B.lib.hc_last_error()
        staging = torch.empty(4 * O.page_payload_bytes(rig.geom), dtype=torch.uint8, device="cuda")
        staged = B.Pool(layers=shape.layers, page_size=shape.page_size, subs=list(shape.subs),
                        device_slots=shape.device_slots, host_pages=shape.host_pages,
                        device_layers=[[rig.dev[b][l] for l in range(shape.layers)] for b in range(len(shape.subs))],
                        host=pair.host_b, stream=rig.stream, staging=staging, write_back_mode=B.HC_MODE_STAGED)
        code = B.lib.hc_write_back_all_layers_noalloc(staged.handle, ctypes.c_void_p(d_t.data_ptr()),
                                                      pair.lists.ptr, n, None)
        assert code == B.HC_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert (pair.host_b.np == FILL).all(), "a refused call changed the host pool"
    finally:
        if staged is not None:
            staged.close()
        pair.close()


@pytest.mark.gpu
def test_no_alloc_write_back_reports_bad_device_rows():
    """The kernels range-check every device slot: an out-of-range slot is skipped and reported
    (HC_ERR_DEVICE with its list position) at the next sync, and every other row lands; with
    HC_FLAG_VALIDATE a page-block list whose rows do not form one whole device page is reported
    the same way."""
    shape = SHAPES[0]
    say("[noalloc] device-side reports")
    pair = Pair(shape, seed=14)
    try:
        rig = pair.rig
        h, d = burst(shape, 6, 500)
        bad_at = 7
        d_bad = d.copy()
        d_bad[bad_at] = shape.device_slots + 5  # out of range
        pair.lists.np.view(np.int64)[:h.size] = h
        dev0 = rig.dev_np()
        torch.cuda.synchronize()
        pair.pool_b.write_back_all_layers_noalloc(cuda_i64(d_bad), pair.lists, h.size)
        with pytest.raises(B.HcError) as e:
            pair.pool_b.sync()
        assert e.value.code == B.HC_ERR_DEVICE and f"position {bad_at}" in str(e.value)
        keep = np.arange(h.size) != bad_at
        want = np.full(pair.host_b.np.size, FILL, dtype=np.uint8)
        O.write_back(rig.geom, dev0, want, d[keep], h[keep])
        assert_bytes_equal(pair.host_b.np, want, "rows other than the bad one")
        pair.pool_b.sync()  # the report was cleared
    finally:
        pair.close()
    blk = SHAPES[2]
    rig = Rig(blk, seed=15, flags=B.HC_FLAG_VALIDATE)
    lists = B.HostBuffer(8 * MAX)
    try:
        h, d = burst(blk, 3, 600)
        P = blk.page_size
        d_mis = d.copy()
        d_mis[P:2 * P] = d[P:2 * P] + 1 if d[2 * P - 1] + 1 < blk.device_slots else d[P:2 * P] - 1  # page 2 shifted
        lists.np.view(np.int64)[:h.size] = h
        torch.cuda.synchronize()
        rig.pool.write_back_all_layers_noalloc(cuda_i64(d_mis), lists, h.size)
        with pytest.raises(B.HcError) as e:
            rig.pool.sync()
        assert e.value.code == B.HC_ERR_DEVICE and "whole device page" in str(e.value)
    finally:
        lists.free()
        rig.close()
