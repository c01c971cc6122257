"""Write-back and load-back at the same time: two pools over the same device and host
buffers, each on its own stream, moving disjoint rows.  Every byte of both pools must
equal what the oracle's write-back and per-layer load-back give on the same inputs
(the bursts touch disjoint rows, so their order does not matter)."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, assert_bytes_equal, assert_dev_equal, cuda_i64, say
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
PF, SH, TM = W.PAGE_FIRST, W.KV_SPLIT_SHARD, W.PAGE_FIRST_TOKEN_MAJOR


def S(name, L, P, subs, slots, pages, layout=PF, align=4096):
    return W.PoolShape(name, L, P, tuple(subs), slots, pages, layout, align)


SHAPES = [
    S("duplex_rows", 4, 64, [(T, 2048)] * 2, 32768, 96),
    S("duplex_indexer", 3, 64, [(T, 1152), (BLK, 8448)], 8192, 48),
    S("duplex_shard_pad", 3, 16, [(T, 1024), (T, 128)], 8192, 96, SH),
    S("duplex_token_major", 4, 16, [(T, 2048), (T, 512)], 8192, 96, TM),
]


def has_blocks(shape):
    return any(g == BLK for g, _ in shape.subs)


def bursts(shape, seed, pages):
    """(write-back slots, host tokens), (load-back host tokens, slots): disjoint host pages,
    disjoint device slots."""
    P = shape.page_size
    all_pages = W.host_pages(seed, shape.host_pages, 2 * pages)
    hw = W.whole_page_tokens(all_pages[:pages], P)
    hl = W.whole_page_tokens(all_pages[pages:], P)
    if shape.layout == SH:
        # a partial last page on the write side: the pad is still written, other rows stay
        hw = hw[:-5]
    if has_blocks(shape):
        dw = W.page_aligned_slots(seed + 1, shape.device_slots, P, hw.size // P)
        dl = W.page_aligned_slots(seed + 2, shape.device_slots, P, hl.size // P, exclude_pages=np.unique(dw // P))
    else:
        dw = W.segment_slots(seed + 1, shape.device_slots, hw.size)
        dl = W.permutation_slots(seed + 2, shape.device_slots, hl.size, exclude=dw)
    return (dw, hw), (hl, dl)


@pytest.mark.gpu
@pytest.mark.parametrize("staged", [True, False], ids=["staged", "zerocopy"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_write_back_and_load_back_at_once(shape, staged):
    say(f"[duplex] {shape.name} staged={staged}")
    rig = Rig(shape, seed=21, staging_pages=3 if staged else 0,
              write_back_mode=B.HC_MODE_STAGED if staged else B.HC_MODE_ZEROCOPY)
    rpool = None
    try:
        L = shape.layers
        rig.host.np[:] = np.random.default_rng(22).integers(0, 256, rig.host.np.size, dtype=np.uint8)
        load_stream = torch.cuda.Stream()
        # staged: the library's duplex pairing; zero-copy: the same grid cap by hand
        rpool = rig.pool.duplex_partner(load_stream) if staged else rig.pool.sibling(load_stream, max_ctas=8)
        for r in range(3):
            (dw, hw), (hl, dl) = bursts(shape, 30 + 10 * r, 9 + 2 * r)
            dw_t, hl_t, dl_t = cuda_i64(dw), cuda_i64(hl), cuda_i64(dl)
            torch.cuda.synchronize()
            dev0 = rig.dev_np()
            host0 = rig.host.np.copy()
            start = B.HipEvent()
            first, second = (rig.stream, load_stream) if r % 2 == 0 else (load_stream, rig.stream)
            start.record(first)
            start.wait_on(second)
            rig.pool.write_back_all_layers(dw_t, hw)
            for l in range(L):
                rpool.load_back_layer(l, hl_t, dl_t)
            rig.pool.sync()
            rpool.sync()
            want_host = host0.copy()
            O.write_back(rig.geom, dev0, want_host, dw, hw)
            want_dev = [[a.copy() for a in row] for row in dev0]
            for l in range(L):
                O.load_back_layer(rig.geom, l, want_dev, host0, hl, dl)
            assert_bytes_equal(rig.host.np, want_host, f"host pool, round {r}")
            assert_dev_equal(rig.dev_np(), want_dev, f"device pool, round {r}")
        if not staged:
            with pytest.raises(ValueError):
                rig.pool.duplex_partner(load_stream)
    finally:
        if rpool is not None:
            rpool.close()
        rig.close()
