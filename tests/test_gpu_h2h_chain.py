"""The storage chain of the shard layout on the GPU, each stage against the oracle
(CacheStore H2H page: Dump path, Load path, page_first_kv_split support).

1. GPU write-back of a burst into a page-first host pool (staged or zero-copy): the
   whole host pool equals orc_write_back's, the device pool is unchanged;
2. hc_h2h dump of the written pages into store shards (1 or 4 CPU workers): the whole
   store equals orc_h2h_dump's (shard pads zero);
3. hc_h2h load of those shards into other host pages: the whole host pool equals
   orc_h2h_load's;
4. per-layer GPU load-back from those other pages into fresh device slots: the whole
   device pool equals orc_load_back_layer's, and every row that went the whole way
   (device -> host -> store -> host -> device) equals the row it started as."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, load_back_and_check, say, write_back_and_check
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
PF = W.PAGE_FIRST

# (name, layers, page size, sub-buffers, device slots, host pages, store shards)
CHAINS = [
    ("kv_pad2048", 3, 16, ((T, 1024), (T, 128)), 4096, 48, 40),     # K 49152 + V 6144 -> 57344: 2048 B pad
    ("kv_aligned", 4, 16, ((T, 2048), (T, 2048)), 8192, 48, 40),     # 262144 B = 64 x 4096: no pad
    ("latent_indexer", 2, 64, ((T, 1152), (BLK, 8448)), 8192, 24, 20),  # 164352 -> 167936: 3584 B pad
]


def has_blocks(subs):
    return any(g == BLK for g, _ in subs)


@pytest.mark.gpu
@pytest.mark.parametrize("workers", [1, 4])
@pytest.mark.parametrize("mode", ["staged", "zerocopy"])
@pytest.mark.parametrize("chain", CHAINS, ids=lambda c: c[0])
def test_write_back_dump_load_load_back(chain, mode, workers):
    name, L, P, subs, S, H, NS = chain
    say(f"[h2h chain] {name} {mode} workers={workers}")
    shape = W.PoolShape(name, L, P, subs, S, H, PF, 4096)
    wb = B.HC_MODE_STAGED if mode == "staged" else B.HC_MODE_ZEROCOPY
    rig = Rig(shape, seed=21, write_back_mode=wb, staging_pages=6 if mode == "staged" else 0)
    eng = None
    try:
        rng = np.random.default_rng([CHAINS.index(chain), int(mode == "staged"), workers])
        npages = 12
        src = rng.choice(H, size=npages, replace=False)
        h = W.whole_page_tokens(src, P)
        if not has_blocks(subs):  # the last page named in part: its other rows keep the fill
            h = h[: h.size - P // 2]
        if has_blocks(subs):
            d = W.page_aligned_slots(int(rng.integers(1 << 30)), S, P, npages)
        else:
            d = rng.choice(S, size=h.size, replace=False).astype(np.int64)
        # 1. write-back (whole host pool and device pool against the oracle)
        write_back_and_check(rig, d, h)

        # 2. dump the written pages into store shards
        pf = rig.geom
        sh = O.Geometry(L, P, list(subs), NS, S, O.KV_SPLIT_SHARD, align=4096)
        stride = O.shard_bytes(sh)
        store = rng.integers(0, 256, O.host_pool_bytes(sh), dtype=np.uint8)
        shards = rng.choice(NS, size=npages, replace=False)
        want_store = store.copy()
        O.h2h_dump(pf, sh, rig.host.np, want_store, src, shards)
        sizes = [O.sub_page_bytes(pf, b) for b in range(len(subs))]
        base = rig.host.ptr.value
        page_ptrs = [[base + O.host_offset(pf, b, int(p), 0, 0) for b in range(len(subs))] for p in src]
        shard_ptrs = [store.ctypes.data + int(q) * stride for q in shards]
        eng = B.H2H(workers=workers, queue_depth=256)
        eng.wait(eng.submit(B.HC_H2H_DUMP, sizes, page_ptrs, shard_ptrs, stride))
        assert np.array_equal(store, want_store), "store after the dump differs from the oracle's"
        if stride > O.page_payload_bytes(sh):
            pads = store.reshape(NS, stride)[shards, O.page_payload_bytes(sh):]
            assert not pads.any(), "a dumped shard's pad is not zero"

        # 3. load the shards into other host pages of the same pool
        free = np.setdiff1d(np.arange(H), src)
        back = rng.choice(free, size=npages, replace=False)
        host_before = rig.host.np.copy()
        want_host = host_before.copy()
        O.h2h_load(pf, sh, want_host, store, shards, back)
        back_ptrs = [[base + O.host_offset(pf, b, int(p), 0, 0) for b in range(len(subs))] for p in back]
        eng.wait(eng.submit(B.HC_H2H_LOAD, sizes, back_ptrs, shard_ptrs, stride))
        assert np.array_equal(rig.host.np, want_host), "host pool after the store load differs from the oracle's"

        # 4. per-layer load-back of the reloaded pages into fresh slots
        page_of = {int(a): int(b) for a, b in zip(src, back)}
        h2 = np.array([page_of[int(x) // P] * P + int(x) % P for x in h], dtype=np.int64)
        if has_blocks(subs):
            used = np.unique(d // P)
            fresh = np.setdiff1d(np.arange(S // P), used)
            dp = rng.choice(fresh, size=npages, replace=False)
            d2 = (dp[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
        else:
            d2 = rng.choice(np.setdiff1d(np.arange(S), d), size=h.size, replace=False).astype(np.int64)
        load_back_and_check(rig, h2, d2)
        assert rig.pool.round_trip_check(cuda_i64(d), cuda_i64(d2)) == 0, "a row changed on its way round"
    finally:
        if eng is not None:
            eng.close()
        rig.close()
        torch.cuda.synchronize()
