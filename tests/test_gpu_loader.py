"""The asynchronous load-back enqueue with a real pool: a consumer stream waits on
each layer through the loader's flags and events and copies the layer's loaded rows,
which must equal the host rows element by element; a failed burst releases its
consumers; the next burst is served."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, say
from oracle import oracle as O

T = W.TOKEN_ROWS
SHAPE = W.PoolShape("loader_rows", 8, 16, ((T, 1024), (T, 512)), 16384, 128)


def host_rows(rig, h, layer):
    """The host rows of `layer` named by h, per sub-buffer (the oracle locates them)."""
    return [np.stack([rig.host.np[o:o + e] for o in O.host_offsets(rig.geom, b, layer, h)])
            for b, (_, e) in enumerate(rig.shape.subs)]


def dev_rows(rig, layer, d_t):
    """The device rows of `layer` at d_t, copied on the current stream (the consumer's)."""
    return [rig.dev[b][layer].view(-1, e)[d_t].clone() for b, (_, e) in enumerate(rig.shape.subs)]


def same_rows(got, want) -> bool:
    return all(np.array_equal(g.cpu().numpy(), w) for g, w in zip(got, want))


@pytest.mark.gpu
@pytest.mark.parametrize("asynchronous", [True, False])
def test_loader_with_consumer_stream(asynchronous):
    say(f"[loader] async={asynchronous}")
    rig = Rig(SHAPE, seed=12)
    loader = None
    try:
        pages = W.host_pages(1, SHAPE.host_pages, 48)
        h = W.whole_page_tokens(pages, SHAPE.page_size)
        d = W.permutation_slots(2, SHAPE.device_slots, h.size)
        rig.pool.write_back_all_layers(cuda_i64(d), h)
        rig.pool.sync()
        d2 = W.permutation_slots(3, SHAPE.device_slots, h.size, exclude=d)
        h_t, d2_t = cuda_i64(h), cuda_i64(d2)
        start = B.HipEvent()
        start.record(torch.cuda.current_stream())  # the index lists are ready on the producer stream
        events = [B.HipEvent() for _ in range(SHAPE.layers)]
        loader = B.Loader(rig.pool, SHAPE.layers, asynchronous=asynchronous)
        burst = loader.submit(h_t, d2_t, h.size, events, start_event=start)
        consumer = torch.cuda.Stream()
        got = []
        for l in range(SHAPE.layers):
            burst.wait_layer(l, consumer)
            with torch.cuda.stream(consumer):
                got.append(dev_rows(rig, l, d2_t))
        consumer.synchronize()
        burst.wait()
        for l in range(SHAPE.layers):
            assert same_rows(got[l], host_rows(rig, h, l)), f"layer {l}"
        # a failing burst (null host list) still completes every layer event
        bad_events = [B.HipEvent() for _ in range(SHAPE.layers)]
        bad = loader.submit(None, d2_t, h.size, bad_events)
        bad.wait_layer(SHAPE.layers - 1, consumer)
        consumer.synchronize()
        with pytest.raises(B.HcError):
            bad.wait()
        assert loader.info()[0] == 1
        # and the next one is served
        good = loader.submit(h_t, d2_t, h.size, events)
        good.wait()
        rig.pool.sync()
        for l in range(SHAPE.layers):
            assert same_rows(dev_rows(rig, l, d2_t), host_rows(rig, h, l))
    finally:
        if loader is not None:
            loader.close()
        rig.close()


@pytest.mark.gpu
def test_loader_and_caller_share_a_pool():
    """A loader thread enqueues one burst's load-back while the calling thread writes
    another burst back on the same pool; both end bit-exact (the pool serializes its
    entry points)."""
    say("[loader] shared pool")
    rig = Rig(SHAPE, seed=16)
    loader = None
    try:
        P = SHAPE.page_size
        pages_a = W.host_pages(5, SHAPE.host_pages, 40)
        h_a = W.whole_page_tokens(pages_a, P)
        d_a = W.permutation_slots(6, SHAPE.device_slots, h_a.size)
        rig.pool.write_back_all_layers(cuda_i64(d_a), h_a)
        rig.pool.sync()
        free_pages = np.setdiff1d(np.arange(SHAPE.host_pages), pages_a)
        pages_b = np.random.default_rng(7).choice(free_pages, 40, replace=False)
        h_b = W.whole_page_tokens(pages_b, P)
        d_b = W.permutation_slots(8, SHAPE.device_slots, h_b.size, exclude=d_a)
        d_a2 = W.permutation_slots(9, SHAPE.device_slots, h_a.size, exclude=np.concatenate([d_a, d_b]))
        dev0 = [[rig.dev[b][l].cpu().numpy() for l in range(SHAPE.layers)] for b in range(2)]
        host0 = rig.host.np.copy()
        loader = B.Loader(rig.pool, SHAPE.layers, asynchronous=True)
        events = [B.HipEvent() for _ in range(SHAPE.layers)]
        bursts = []
        for _ in range(4):  # several bursts so the worker runs while the caller writes back
            bursts.append(loader.submit(cuda_i64(h_a), cuda_i64(d_a2), h_a.size, events))
            rig.pool.write_back_all_layers(cuda_i64(d_b), h_b)
        for bu in bursts:
            bu.wait()
        rig.pool.sync()
        want_host = host0.copy()
        O.write_back(rig.geom, dev0, want_host, d_b, h_b)
        assert np.array_equal(rig.host.np, want_host), "write-back under a busy loader differs"
        for l in range(SHAPE.layers):
            O.load_back_layer(rig.geom, l, dev0, host0, h_a, d_a2)
        for b in range(2):
            for l in range(SHAPE.layers):
                assert np.array_equal(rig.dev[b][l].cpu().numpy(), dev0[b][l]), (b, l)
    finally:
        if loader is not None:
            loader.close()
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("asynchronous", [True, False])
def test_loader_replays_a_captured_burst(asynchronous):
    """Captured bursts handed to the loader: each replay follows the index buffers, a
    consumer waits per layer through the loader, and replays queue behind eager bursts."""
    say(f"[loader] captured bursts async={asynchronous}")
    rig = Rig(SHAPE, seed=13)
    loader = graph = None
    try:
        pages = W.host_pages(4, SHAPE.host_pages, 40)
        h = W.whole_page_tokens(pages, SHAPE.page_size)
        d = W.permutation_slots(5, SHAPE.device_slots, h.size)
        rig.pool.write_back_all_layers(cuda_i64(d), h)
        rig.pool.sync()
        h_t = cuda_i64(h)
        d_buf = cuda_i64(W.permutation_slots(6, SHAPE.device_slots, h.size, exclude=d))
        events = [B.HipEvent() for _ in range(SHAPE.layers)]
        graph = rig.pool.capture_load_back(h_t, d_buf, events)
        loader = B.Loader(rig.pool, SHAPE.layers, asynchronous=asynchronous)
        consumer = torch.cuda.Stream()
        for r in range(3):
            d2 = W.permutation_slots(10 + r, SHAPE.device_slots, h.size, exclude=d)
            d_buf.copy_(cuda_i64(d2))
            start = B.HipEvent()
            start.record(torch.cuda.current_stream())  # the rewritten slot list is ready
            burst = loader.submit_graph(graph, events, start_event=start)
            got = []
            for l in range(SHAPE.layers):
                burst.wait_layer(l, consumer)
                with torch.cuda.stream(consumer):
                    got.append(dev_rows(rig, l, d_buf))
            consumer.synchronize()
            burst.wait()
            burst.release()
            for l in range(SHAPE.layers):
                assert same_rows(got[l], host_rows(rig, h, l)), f"replay {r} layer {l}"
            # an eager burst between replays, on other events
            other = [B.HipEvent() for _ in range(SHAPE.layers)]
            eager = loader.submit(h_t, cuda_i64(d2), h.size, other)
            eager.wait()
            eager.release()
        rig.pool.sync()
    finally:
        if loader is not None:
            loader.close()
        if graph is not None:
            graph.close()
        rig.close()


@pytest.mark.gpu
def test_loader_refuses_a_graph_it_could_not_flag():
    """With the pool's own ops, a captured burst is handed over only with the exact events it
    records and only to a loader of its own pool; anything else would leave a consumer
    waiting on an event no replay records."""
    say("[loader] mismatched captured bursts refused")
    rig = Rig(SHAPE, seed=14)
    other_rig = Rig(SHAPE, seed=15)
    loader = None
    graphs = []
    try:
        h = W.whole_page_tokens(W.host_pages(7, SHAPE.host_pages, 4), SHAPE.page_size)
        d = W.permutation_slots(8, SHAPE.device_slots, h.size)
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        events = [B.HipEvent() for _ in range(SHAPE.layers)]
        g = rig.pool.capture_load_back(h_t, d_t, events)
        graphs.append(g)
        with_gap = list(events)
        with_gap[2] = None
        g_gap = rig.pool.capture_load_back(h_t, d_t, with_gap)
        graphs.append(g_gap)
        g_other = other_rig.pool.capture_load_back(h_t, d_t, events)
        graphs.append(g_other)
        loader = B.Loader(rig.pool, SHAPE.layers, asynchronous=True)
        swapped = list(events)
        swapped[3], swapped[4] = swapped[4], swapped[3]
        cases = [(g, swapped, "layer 3"), (g, [B.HipEvent() for _ in events], "layer 0"),
                 (g_gap, events, "layer 2"), (g_other, events, "another pool")]
        for graph, evs, why in cases:
            with pytest.raises(B.HcError) as ex:
                loader.submit_graph(graph, evs)
            assert ex.value.code == B.HC_ERR_INVALID and why in str(ex.value), str(ex.value)
        with pytest.raises(ValueError):
            loader.submit_graph(g, events[:-1])
        # nothing was queued by the refusals; the matching hand-over still runs
        burst = loader.submit_graph(g, events)
        assert burst.wait() is None
        burst.release()
        assert loader.info() == (0, True)
    finally:
        if loader is not None:
            loader.close()
        for graph in graphs:
            graph.close()
        other_rig.close()
        rig.close()


@pytest.mark.gpu
def test_start_event_orders_the_producers_index_list_before_the_burst():
    """The producer writes the slot list on its own stream after a bounded spin and records
    the start event; the loader's transfer stream waits on it, so the kernels read the new
    list, not the sentinel the buffer held before (loader-thread page, Modifications: the
    index move runs after the start-event wait).  Negative control: without the start
    event the same burst reads the sentinel, so the check has teeth."""
    say("[loader] start event orders the index list")
    rig = Rig(SHAPE, seed=16)
    loader = None
    try:
        L, n_pages = SHAPE.layers, 24
        h = W.whole_page_tokens(W.host_pages(21, SHAPE.host_pages, n_pages), SHAPE.page_size)
        d = W.permutation_slots(22, SHAPE.device_slots, h.size)
        rig.pool.write_back_all_layers(cuda_i64(d), h)
        rig.pool.sync()
        used = d
        lists = []
        for seed in (23, 24, 25, 26):  # real and sentinel lists of the two runs, all disjoint
            lists.append(W.permutation_slots(seed, SHAPE.device_slots, h.size, exclude=used))
            used = np.concatenate([used, lists[-1]])
        h_t = cuda_i64(h)
        producer = torch.cuda.Stream()
        loader = B.Loader(rig.pool, L, asynchronous=True)
        for k, use_start in enumerate((True, False)):
            real, sentinel = lists[2 * k], lists[2 * k + 1]
            real_t, d_buf = cuda_i64(real), cuda_i64(sentinel)  # the buffer holds the sentinel at hand-over
            events = [B.HipEvent() for _ in range(L)]
            start = B.HipEvent()
            torch.cuda.synchronize()
            producer.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(producer):
                torch.cuda._sleep(50_000_000)  # bounded spin: the producer is still writing the list
                d_buf.copy_(real_t)
                start.record(producer)
            burst = loader.submit(h_t, d_buf, h.size, events, start_event=start if use_start else None)
            burst.wait()
            burst.release()
            torch.cuda.synchronize()
            at_real = all(same_rows(dev_rows(rig, l, real_t), host_rows(rig, h, l)) for l in range(L))
            if use_start:
                assert at_real, "the burst did not wait for the producer's start event"
            else:
                assert not at_real, "negative control: the burst without a start event read the new list anyway"
        rig.pool.sync()
    finally:
        if loader is not None:
            loader.close()
        rig.close()
