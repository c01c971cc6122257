"""Captured load-back bursts (hc_load_back_graph_*) against the oracle.

A graph is captured once per (index buffers, n, events); every replay must do what
the oracle's per-layer load-back does with the index lists the buffers hold at
replay time.  Each test replays several times with new list contents, with eager
library work and synchronizations between replays, and checks every replay."""
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
    W.SHAPES["tiny_mha_bf16"],
    S("graph_indexer", 3, 64, [(T, 1152), (BLK, 8448)], 8192, 32),
    S("graph_shard_pad", 3, 16, [(T, 1024), (T, 128)], 4096, 40, SH),
    S("graph_token_major", 4, 16, [(T, 2048), (T, 2048)], 8192, 64, TM),
]


def has_blocks(shape):
    return any(g == BLK for g, _ in shape.subs)


def lists(shape, pages, seed):
    """(host tokens, device slots) of `pages` whole host pages; page-aligned slots with page blocks."""
    P = shape.page_size
    h = W.whole_page_tokens(W.host_pages(seed, shape.host_pages, pages), P)
    if has_blocks(shape):
        d = W.page_aligned_slots(seed + 1, shape.device_slots, P, pages)
    else:
        d = W.permutation_slots(seed + 1, shape.device_slots, h.size)
    return h, d


def randomize_host(rig, seed):
    rig.host.np[:] = np.random.default_rng(seed).integers(0, 256, rig.host.np.size, dtype=np.uint8)


@pytest.mark.gpu
@pytest.mark.parametrize("pages", [1, 7])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_replays_follow_the_index_buffers(shape, pages):
    say(f"[graph] {shape.name} pages={pages}")
    rig = Rig(shape, seed=3)
    graph = None
    try:
        randomize_host(rig, 5)
        L = shape.layers
        h0, d0 = lists(shape, pages, 10)
        h_buf, d_buf = cuda_i64(h0), cuda_i64(d0)
        events = [B.HipEvent() for _ in range(L)]
        torch.cuda.synchronize()
        before = rig.dev_np()
        graph = rig.pool.capture_load_back(h_buf, d_buf, events)
        # capture enqueues nothing: the device pool is unchanged until a replay
        rig.pool.sync()
        assert_dev_equal(rig.dev_np(), before, "capture moved rows")
        for r in range(3):
            h, d = lists(shape, pages, 20 + 7 * r)
            h_buf.copy_(cuda_i64(h))
            d_buf.copy_(cuda_i64(d))
            torch.cuda.synchronize()
            dev0 = rig.dev_np()
            host0 = rig.host.np.copy()
            graph.launch()
            for ev in events:
                ev.synchronize()
            rig.pool.sync()
            want = [[a.copy() for a in row] for row in dev0]
            for l in range(L):
                O.load_back_layer(rig.geom, l, want, host0, h, d)
            assert_dev_equal(rig.dev_np(), want, f"replay {r}")
            assert_bytes_equal(rig.host.np, host0, f"host pool changed by replay {r}")
            # eager library work between replays
            e = cuda_i64(np.empty(0, dtype=np.int64))
            rig.pool.load_back_layer(0, e, e)
            assert rig.pool.round_trip_check(cuda_i64(d), cuda_i64(d)) == 0
        graph.close()
        graph = None
    finally:
        if graph is not None:
            graph.close()
        rig.close()


@pytest.mark.gpu
def test_replay_layer_events_release_a_consumer():
    """A consumer stream that waits on each layer event of a replay sees that layer's rows."""
    shape = S("graph_consumer", 6, 16, [(T, 1024), (T, 1024)], 8192, 64)
    say("[graph] consumer")
    rig = Rig(shape, seed=4)
    graph = None
    try:
        randomize_host(rig, 6)
        L, P = shape.layers, shape.page_size
        h, d = lists(shape, 12, 30)
        h_buf, d_buf = cuda_i64(h), cuda_i64(d)
        events = [B.HipEvent() for _ in range(L)]
        graph = rig.pool.capture_load_back(h_buf, d_buf, events)
        consumer = torch.cuda.Stream()
        host0 = rig.host.np.copy()
        for r in range(2):
            torch.cuda.synchronize()
            got = []
            graph.launch()
            for l in range(L):
                events[l].wait_on(consumer)
                with torch.cuda.stream(consumer):
                    got.append([rig.dev[b][l].view(-1, e)[d_buf].clone() for b, (_, e) in enumerate(shape.subs)])
            torch.cuda.synchronize()
            for l in range(L):
                for b in range(len(shape.subs)):
                    offs = O.host_offsets(rig.geom, b, l, h)
                    e = shape.subs[b][1]
                    want = host0[(offs[:, None] + np.arange(e)[None, :])]
                    assert np.array_equal(got[l][b].cpu().numpy(), want), f"replay {r} layer {l} sub {b}"
    finally:
        if graph is not None:
            graph.close()
        rig.close()


@pytest.mark.gpu
def test_empty_burst_graph_records_events_only():
    shape = SHAPES[0]
    say("[graph] empty")
    rig = Rig(shape, seed=7)
    graph = None
    try:
        e = cuda_i64(np.empty(0, dtype=np.int64))
        events = [B.HipEvent() for _ in range(shape.layers)]
        events[1] = None
        graph = rig.pool.capture_load_back(e, e, events)
        dev0 = rig.dev_np()
        graph.launch()
        for ev in events:
            if ev is not None:
                ev.synchronize()
        rig.pool.sync()
        assert_dev_equal(rig.dev_np(), dev0, "empty replay changed the device pool")
    finally:
        if graph is not None:
            graph.close()
        rig.close()


@pytest.mark.gpu
def test_profiling_pool_is_refused():
    shape = SHAPES[0]
    say("[graph] profiling refused")
    rig = Rig(shape, seed=8, flags=B.HC_FLAG_PROFILE)
    try:
        h, d = lists(shape, 2, 40)
        with pytest.raises(B.HcError) as ex:
            rig.pool.capture_load_back(cuda_i64(h), cuda_i64(d), [B.HipEvent() for _ in range(shape.layers)])
        assert ex.value.code == B.HC_ERR_UNSUPPORTED
        # the stream is not left capturing: eager calls still work
        rig.pool.load_back_layer(0, cuda_i64(h), cuda_i64(d))
        rig.pool.sync()
    finally:
        rig.close()


@pytest.mark.gpu
def test_replay_with_an_out_of_range_slot_is_reported_not_faulted():
    """Kernels range-check device-resident indices, in a replay as eagerly: the bad row is
    skipped, the others land, and the next sync reports HC_ERR_DEVICE."""
    shape = SHAPES[0]
    say("[graph] out-of-range slot in a replay")
    rig = Rig(shape, seed=9)
    graph = None
    try:
        randomize_host(rig, 11)
        L = shape.layers
        h, d = lists(shape, 3, 50)
        h_buf, d_buf = cuda_i64(h), cuda_i64(d)
        events = [B.HipEvent() for _ in range(L)]
        graph = rig.pool.capture_load_back(h_buf, d_buf, events)
        bad = d.copy()
        bad[4] = shape.device_slots + 3
        d_buf.copy_(cuda_i64(bad))
        torch.cuda.synchronize()
        dev0 = rig.dev_np()
        host0 = rig.host.np.copy()
        graph.launch()
        for ev in events:
            ev.synchronize()
        with pytest.raises(B.HcError) as ex:
            rig.pool.sync()
        assert ex.value.code == B.HC_ERR_DEVICE and "out of range" in str(ex.value)
        assert "first flagged list position 4)" in str(ex.value), str(ex.value)
        rig.pool.sync()  # the report is cleared once read
        keep = np.arange(h.size) != 4
        want = [[a.copy() for a in row] for row in dev0]
        for l in range(L):
            O.load_back_layer(rig.geom, l, want, host0, h[keep], bad[keep])
        assert_dev_equal(rig.dev_np(), want, "replay with one bad slot")
    finally:
        if graph is not None:
            graph.close()
        rig.close()


@pytest.mark.gpu
def test_pool_outlives_its_graphs_and_loaders():
    """hc_pool_destroy refuses while a captured graph or a loader still holds the pool."""
    shape = SHAPES[0]
    say("[graph] pool destroy refused while held")
    rig = Rig(shape, seed=12)
    try:
        h, d = lists(shape, 2, 60)
        graph = rig.pool.capture_load_back(cuda_i64(h), cuda_i64(d), [B.HipEvent() for _ in range(shape.layers)])
        loader = B.Loader(rig.pool, shape.layers, asynchronous=True)
        with pytest.raises(B.HcError) as ex:
            rig.pool.close()
        assert ex.value.code == B.HC_ERR_INVALID and "destroy them first" in str(ex.value)
        graph.close()
        with pytest.raises(B.HcError):
            rig.pool.close()
        loader.close()
        rig.pool.load_back_layer(0, cuda_i64(h), cuda_i64(d))  # the pool still works
        rig.pool.sync()
    finally:
        rig.close()


@pytest.mark.gpu
def test_caller_capture_rules_on_a_profiling_pool():
    """A caller's own capture on the pool's stream.  The write-back (its plan is built on the
    CPU per call), hc_pool_sync and hc_round_trip_check (they wait for the stream), creating a
    pool on the capturing stream (its set-up copies and waits) and destroying one (it waits
    before freeing) are refused with HC_ERR_UNSUPPORTED and leave the capture usable (the
    refused pool is destroyed after the capture); per-layer load-backs and a layer pack
    recorded on a profiling pool are not timed, and every replay (host pool rewritten between
    replays) matches the oracle."""
    shape = SHAPES[1]
    say("[graph] caller capture on a profiling pool")
    rig = Rig(shape, seed=9, flags=B.HC_FLAG_PROFILE)
    try:
        L = shape.layers
        h, d = lists(shape, 5, 60)
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        staging = torch.zeros(rig.pool.layer_pack_bytes(d.size), dtype=torch.uint8, device="cuda")
        rig.pool.kernel_time(B.KIND_ZC_READ, reset=True)
        other = rig.pool.sibling(rig.stream)
        torch.cuda.synchronize()
        refused = {}
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=rig.stream, capture_error_mode="thread_local"):
            for what, call in (("write-back", lambda: rig.pool.write_back_all_layers(d_t, h)),
                               ("sync", rig.pool.sync),
                               ("round-trip check", lambda: rig.pool.round_trip_check(d_t, d_t)),
                               ("pool create", lambda: rig.pool.sibling(rig.stream)),
                               ("pool destroy", other.close)):
                try:
                    call()
                except B.HcError as e:
                    refused[what] = e.code
            for l in range(L):
                rig.pool.load_back_layer(l, h_t, d_t)
            rig.pool.layer_pack(L - 1, d_t, staging)
        assert refused == {"write-back": B.HC_ERR_UNSUPPORTED, "sync": B.HC_ERR_UNSUPPORTED,
                           "round-trip check": B.HC_ERR_UNSUPPORTED, "pool create": B.HC_ERR_UNSUPPORTED,
                           "pool destroy": B.HC_ERR_UNSUPPORTED}, refused
        assert other.handle.value, "the refused destroy freed the pool"
        other.close()
        torch.cuda.synchronize()
        for replay in range(3):
            randomize_host(rig, 70 + replay)
            dev0, host0 = rig.dev_np(), rig.host.np.copy()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            rig.pool.sync()
            want = [[a.copy() for a in row] for row in dev0]
            for l in range(L):
                O.load_back_layer(rig.geom, l, want, host0, h, d)
            assert_dev_equal(rig.dev_np(), want, f"device pool after replay {replay}")
            packed = O.layer_pack(rig.geom, L - 1, want, d)
            assert_bytes_equal(staging.cpu().numpy(), packed, f"pack staging after replay {replay}")
            assert rig.pool.round_trip_check(d_t, d_t) == 0
        launches, _ = rig.pool.kernel_time(B.KIND_ZC_READ)
        assert launches == 0, "a recorded launch was timed"
        rig.pool.load_back_layer(0, h_t, d_t)  # eager again: timed
        launches, _ = rig.pool.kernel_time(B.KIND_ZC_READ)
        assert launches == 1
        del graph
    finally:
        rig.close()
