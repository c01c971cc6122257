"""Back-to-back bursts on one pool with no synchronisation in between: write-backs of
random sizes (the plan buffers alternate and grow while earlier bursts are still queued)
and per-layer load-backs, some naming host pages an earlier burst of the run wrote.
Temporaries are passed on purpose.  After one final sync the whole host pool and device
pool must equal the oracle applied to the same calls in the same order."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, assert_bytes_equal, assert_dev_equal, cuda_i64, say
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
PF, SH, TM = W.PAGE_FIRST, W.KV_SPLIT_SHARD, W.PAGE_FIRST_TOKEN_MAJOR
SHAPES = [
    W.PoolShape("stress_rows", 3, 16, ((T, 256), (T, 128)), 4096, 96, PF),
    W.PoolShape("stress_shard", 2, 8, ((T, 512), (T, 96)), 2048, 80, SH, 1024),
    W.PoolShape("stress_blocks", 2, 16, ((T, 64), (BLK, 512)), 2048, 64, TM),
]


@pytest.mark.gpu
@pytest.mark.parametrize("staged", [False, True], ids=["zerocopy", "staged"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_back_to_back_bursts_without_sync(shape, staged):
    say(f"[stress] {shape.name} staged={staged}")
    P, L, S, H = shape.page_size, shape.layers, shape.device_slots, shape.host_pages
    blocks = any(g == BLK for g, _ in shape.subs)
    rig = Rig(shape, seed=91, staging_pages=2 if staged else 0,
              write_back_mode=B.HC_MODE_STAGED if staged else B.HC_MODE_ZEROCOPY)
    try:
        rng = np.random.default_rng(92)
        rig.host.np[:] = rng.integers(0, 256, rig.host.np.size, dtype=np.uint8)
        torch.cuda.synchronize()
        dev = rig.dev_np()
        host = rig.host.np.copy()
        for k in range(60):
            npages = int(rng.choice([1, 2, 3, 7, 20, 40]))
            pages = rng.choice(H, size=npages, replace=False)
            if blocks:
                h = W.whole_page_tokens(pages, P)
                dp = rng.choice(S // P, size=npages, replace=False)
                d = (dp[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
            else:
                h = np.concatenate([p * P + np.sort(rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False))
                                    for p in pages]).astype(np.int64)
                d = rng.choice(S, size=h.size, replace=False).astype(np.int64)
            if k % 3 == 2:
                # per-layer load-back of these host rows (some written earlier in the run)
                for l in range(L):
                    rig.pool.load_back_layer(l, cuda_i64(h), cuda_i64(d))
                    O.load_back_layer(rig.geom, l, dev, host, h, d)
            else:
                rig.pool.write_back_all_layers(cuda_i64(d), h)
                O.write_back(rig.geom, dev, host, d, h)
        rig.pool.sync()
        assert_bytes_equal(rig.host.np, host, "host pool after the run")
        assert_dev_equal(rig.dev_np(), dev, "device pool after the run")
    finally:
        rig.close()


@pytest.mark.gpu
def test_one_pool_called_from_several_threads():
    """Four Python threads call one pool at the same time (the library serialises the calls
    on its copy stream): two write back their own host pages, two load back their own
    earlier-written pages into their own slots.  Rows are disjoint between threads, so the
    final pools equal the oracle whatever the interleaving."""
    import threading
    shape = SHAPES[0]
    P, L, S, H = shape.page_size, shape.layers, shape.device_slots, shape.host_pages
    say("[stress] one pool, four threads")
    rig = Rig(shape, seed=93)
    try:
        rng = np.random.default_rng(94)
        rig.host.np[:] = rng.integers(0, 256, rig.host.np.size, dtype=np.uint8)
        torch.cuda.synchronize()
        dev, host = rig.dev_np(), rig.host.np.copy()
        page_sets = np.array_split(rng.permutation(H), 4)
        slot_sets = np.array_split(rng.permutation(S), 4)
        plans = []
        for t in range(4):
            calls = []
            for k in range(25):
                pages = rng.choice(page_sets[t], size=3, replace=False)
                h = W.whole_page_tokens(pages, P)
                d = rng.choice(slot_sets[t], size=h.size, replace=False).astype(np.int64)
                calls.append((h, d))
            plans.append(calls)
        errors = []

        def writer(t):
            try:
                for h, d in plans[t]:
                    rig.pool.write_back_all_layers(cuda_i64(d), h)
            except Exception as e:  # reported below
                errors.append(e)

        def loader(t):
            try:
                for h, d in plans[t]:
                    for l in range(L):
                        rig.pool.load_back_layer(l, cuda_i64(h), cuda_i64(d))
            except Exception as e:
                errors.append(e)

        threads = [threading.Thread(target=writer, args=(0,)), threading.Thread(target=writer, args=(1,)),
                   threading.Thread(target=loader, args=(2,)), threading.Thread(target=loader, args=(3,))]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        assert not errors, errors
        rig.pool.sync()
        for t in (0, 1):
            for h, d in plans[t]:
                O.write_back(rig.geom, dev, host, d, h)
        for t in (2, 3):
            for h, d in plans[t]:
                for l in range(L):
                    O.load_back_layer(rig.geom, l, dev, host, h, d)
        assert_bytes_equal(rig.host.np, host, "host pool")
        assert_dev_equal(rig.dev_np(), dev, "device pool")
    finally:
        rig.close()


@pytest.mark.gpu
def test_profiling_pool_over_many_launches():
    """A pool with per-launch timing folds its pending timing events into the totals every
    4096 launches; 4500 layer launches must all be counted, with every row correct."""
    shape = SHAPES[0]
    P, L, S, H = shape.page_size, shape.layers, shape.device_slots, shape.host_pages
    say("[stress] profiling pool, 4500 launches")
    rig = Rig(shape, seed=97, flags=B.HC_FLAG_PROFILE)
    try:
        rng = np.random.default_rng(98)
        rig.host.np[:] = rng.integers(0, 256, rig.host.np.size, dtype=np.uint8)
        h = W.whole_page_tokens(rng.choice(H, size=2, replace=False), P)
        d = rng.choice(S, size=h.size, replace=False).astype(np.int64)
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        torch.cuda.synchronize()
        dev = rig.dev_np()
        rig.pool.kernel_time(B.KIND_ZC_READ, reset=True)
        for k in range(1500):
            for l in range(L):
                rig.pool.load_back_layer(l, h_t, d_t)
        rig.pool.sync()
        n, ms = rig.pool.kernel_time(B.KIND_ZC_READ)
        assert n == 1500 * L and ms > 0
        for l in range(L):
            O.load_back_layer(rig.geom, l, dev, rig.host.np, h, d)
        assert_dev_equal(rig.dev_np(), dev, "device pool")
    finally:
        rig.close()


@pytest.mark.gpu
def test_pool_stats_count_enqueued_calls():
    """hc_pool_get_stats: calls, tokens and host-link bytes of enqueued write-backs and
    per-layer load-backs (captured replays included, refused calls not), and device
    error reports."""
    shape = SHAPES[2]  # token rows plus page blocks
    P, L, S, H = shape.page_size, shape.layers, shape.device_slots, shape.host_pages
    rows = sum(e for g, e in shape.subs if g == T)
    blks = sum(e for g, e in shape.subs if g == BLK)
    say("[stress] pool stats")
    rig = Rig(shape, seed=99)
    graph = None
    try:
        rng = np.random.default_rng(100)
        pages = rng.choice(H, size=5, replace=False)
        h = W.whole_page_tokens(pages, P)
        dp = rng.choice(S // P, size=5, replace=False)
        d = (dp[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
        n = h.size
        assert rig.pool.stats() == {f: 0 for f, _ in B.hc_pool_stats._fields_}
        rig.pool.write_back_all_layers(cuda_i64(d), h)
        with pytest.raises(B.HcError):
            rig.pool.write_back_all_layers(cuda_i64(d), h[::-1].copy())  # rows out of order: refused
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        for l in range(L):
            rig.pool.load_back_layer(l, h_t, d_t)
        graph = rig.pool.capture_load_back(h_t, d_t, [B.HipEvent() for _ in range(L)])
        graph.launch()
        graph.launch()
        bad = d.copy()
        bad[0] = S * 4  # out of range: skipped and reported
        rig.pool.load_back_layer(0, h_t, cuda_i64(bad))
        with pytest.raises(B.HcError):
            rig.pool.sync()
        per_layer = n * rows + (n // P) * blks
        st = rig.pool.stats()
        assert st["write_back_calls"] == 1 and st["write_back_tokens"] == n
        assert st["write_back_bytes"] == per_layer * L
        assert st["load_back_calls"] == L + 2 * L + 1
        assert st["load_back_tokens"] == n * (3 * L + 1)
        assert st["load_back_bytes"] == per_layer * (3 * L + 1)
        assert st["device_errors"] == 1
    finally:
        if graph is not None:
            graph.close()
        rig.close()
