"""A serving-shaped loop over the whole path.  Each round a staged write-back of one
request's pages (pool A, copy stream A) runs while a loader thread loads back, layer by
layer, pages an earlier round wrote (pool B, a sibling over the same buffers on stream B,
8 workgroups), and a consumer stream waits on each layer-done event and checksums the
layer.  Every round checks the written host pages byte for byte against the device rows
they came from, and every consumed layer against the host rows it was loaded from.

The device index lists are passed as temporaries on purpose: the binding must keep torch's
caching allocator from handing their memory to the next allocation while the pool's copy
stream still reads them (without that, the last staging chunk of a round gathered the
wrong rows)."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, say
from oracle import oracle as O

T = W.TOKEN_ROWS
SHAPE = W.PoolShape("serving_loop", 6, 16, ((T, 512), (T, 512)), 16384, 256)


def host_rows(rig, b, layer, h):
    e = SHAPE.subs[b][1]
    offs = O.host_offsets(rig.geom, b, layer, h)
    return rig.host.np[(offs[:, None] + np.arange(e)[None, :])]


@pytest.mark.gpu
def test_write_back_beside_loader_driven_load_back_with_consumer():
    say("[serving loop] 6 rounds")
    L, P = SHAPE.layers, SHAPE.page_size
    rig = Rig(SHAPE, seed=81, staging_pages=4, write_back_mode=B.HC_MODE_STAGED)
    loader = None
    bpool = None
    try:
        bpool = rig.pool.sibling(torch.cuda.Stream(), max_ctas=8)
        loader = B.Loader(bpool, L, asynchronous=True)
        consumer = torch.cuda.Stream()
        rng = np.random.default_rng(82)
        free_pages = list(rng.permutation(SHAPE.host_pages))
        written = []          # host pages of earlier rounds, with their host tokens
        busy_slots = np.empty(0, dtype=np.int64)
        for r in range(6):
            # this round's request: 5 fresh host pages, whose rows sit in random device slots
            pages = np.array([free_pages.pop() for _ in range(5)])
            h_w = W.whole_page_tokens(pages, P)
            d_w = W.permutation_slots(100 + r, SHAPE.device_slots, h_w.size, exclude=busy_slots)
            # an earlier request's pages come back into fresh slots
            h_l = written[r - 1] if r > 0 else None
            if h_l is not None:
                d_l = W.permutation_slots(200 + r, SHAPE.device_slots, h_l.size,
                                          exclude=np.concatenate([busy_slots, d_w]))
            torch.cuda.synchronize()
            want_w = [[rig.dev[b][l].view(-1, e)[cuda_i64(d_w)].cpu().numpy() for l in range(L)]
                      for b, (_, e) in enumerate(SHAPE.subs)]
            want_l = None
            if h_l is not None:
                want_l = [[host_rows(rig, b, l, h_l).copy() for l in range(L)] for b in range(len(SHAPE.subs))]
            # the two directions at once
            rig.pool.write_back_all_layers(cuda_i64(d_w), h_w)
            got = []
            if h_l is not None:
                d_l_t = cuda_i64(d_l)
                start = B.HipEvent()
                start.record(torch.cuda.current_stream())
                events = [B.HipEvent() for _ in range(L)]
                burst = loader.submit(cuda_i64(h_l), d_l_t, h_l.size, events, start_event=start)
                for l in range(L):
                    burst.wait_layer(l, consumer)
                    with torch.cuda.stream(consumer):
                        got.append([rig.dev[b][l].view(-1, e)[d_l_t].clone() for b, (_, e) in enumerate(SHAPE.subs)])
                consumer.synchronize()
                burst.wait()
                burst.release()
            rig.pool.sync()
            bpool.sync()
            # written pages: every row equals the device row it came from
            for b in range(len(SHAPE.subs)):
                for l in range(L):
                    got_w = host_rows(rig, b, l, h_w)
                    if not np.array_equal(got_w, want_w[b][l]):
                        bad = np.flatnonzero((got_w != want_w[b][l]).any(axis=1))
                        now = rig.dev[b][l].view(-1, SHAPE.subs[b][1])[cuda_i64(d_w)].cpu().numpy()
                        raise AssertionError(
                            f"round {r} write sub {b} layer {l}: {bad.size} of {h_w.size} rows differ "
                            f"(first {bad[:8].tolist()}); host equals the device rows now: {np.array_equal(got_w, now)}; "
                            f"device rows changed since the snapshot: {not np.array_equal(now, want_w[b][l])}; "
                            f"host rows still 0xA5: {int((got_w[bad] == 0xA5).all(axis=1).sum())}")
            # consumed layers: what the consumer saw after each layer event equals the host rows
            for l in range(len(got)):
                for b in range(len(SHAPE.subs)):
                    assert np.array_equal(got[l][b].cpu().numpy(), want_l[b][l]), f"round {r} load sub {b} layer {l}"
            written.append(h_w)
            busy_slots = np.concatenate([busy_slots, d_w] + ([d_l] if h_l is not None else []))
        assert loader.info()[0] == 0
    finally:
        if loader is not None:
            loader.close()
        if bpool is not None:
            bpool.close()
        rig.close()
