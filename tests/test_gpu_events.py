"""Layer-done event chain and failure handling on the GPU (small pools).

- a consumer stream that waits on each layer's event sees exactly the oracle's rows;
- negative control: a consumer that does not wait, while the copy stream is held
  back by a bounded spin, sees stale rows (so the positive check has teeth);
- a failing load-back call still records its event, so a waiting consumer is
  released (the loader-failure rule of the loader-thread page, Modifications);
- bad indices are rejected on the host (write-back) or skipped and reported by the
  kernels' own range checks (load-back), never dereferenced."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, say, write_back_and_check
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
SHAPE = W.PoolShape("event_rows", 6, 16, ((T, 1024), (T, 1024)), 16384, 128)
BLOCKS = W.PoolShape("event_blocks", 3, 16, ((T, 64), (BLK, 256)), 4096, 64)


def expected_layer_rows(rig, h, layer):
    """The host rows of `layer` named by h, per sub-buffer (the oracle locates them)."""
    return [np.stack([rig.host.np[o:o + e] for o in O.host_offsets(rig.geom, b, layer, h)])
            for b, (gran, e) in enumerate(rig.shape.subs)]


def consumer_rows(rig, layer, d_t):
    """The device rows of `layer` at d_t, copied on the current stream (the consumer's)."""
    return [rig.dev[b][layer].view(-1, e)[d_t].clone() for b, (gran, e) in enumerate(rig.shape.subs)]


def same_rows(got, want) -> bool:
    return all(np.array_equal(g.cpu().numpy(), w) for g, w in zip(got, want))


def prepare(rig, seed):
    """Write a burst back, so the host pool holds known rows, and pick fresh slots."""
    pages = W.host_pages(seed, rig.shape.host_pages, 40)
    h = W.whole_page_tokens(pages, rig.shape.page_size)
    d = W.permutation_slots(seed + 1, rig.shape.device_slots, h.size)
    rig.pool.write_back_all_layers(cuda_i64(d), h)
    rig.pool.sync()
    d2 = W.permutation_slots(seed + 2, rig.shape.device_slots, h.size, exclude=d)
    return h, d, d2


@pytest.mark.gpu
def test_consumer_waits_on_each_layer_event():
    say("[events] consumer with waits")
    rig = Rig(SHAPE, seed=7)
    try:
        h, d, d2 = prepare(rig, 3)
        h_t, d2_t = cuda_i64(h), cuda_i64(d2)
        consumer = torch.cuda.Stream()
        events = [B.HipEvent() for _ in range(SHAPE.layers)]
        torch.cuda.synchronize()
        with torch.cuda.stream(rig.stream):
            torch.cuda._sleep(10_000_000)  # hold the copy stream back; the waits must cover it
        got = []
        for l in range(SHAPE.layers):
            rig.pool.load_back_layer(l, h_t, d2_t, events[l])
            events[l].wait_on(consumer)
            with torch.cuda.stream(consumer):
                got.append(consumer_rows(rig, l, d2_t))
        consumer.synchronize()
        rig.pool.sync()
        for l in range(SHAPE.layers):
            assert same_rows(got[l], expected_layer_rows(rig, h, l)), f"layer {l}"
    finally:
        rig.close()


@pytest.mark.gpu
def test_negative_control_consumer_without_wait_sees_stale_rows():
    say("[events] negative control")
    rig = Rig(SHAPE, seed=8)
    try:
        h, d, d2 = prepare(rig, 5)
        h_t, d2_t = cuda_i64(h), cuda_i64(d2)
        consumer = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(rig.stream):
            torch.cuda._sleep(50_000_000)  # bounded spin
        rig.pool.load_back_layer(0, h_t, d2_t, None)
        with torch.cuda.stream(consumer):
            early = consumer_rows(rig, 0, d2_t)  # no wait: runs while the copy stream spins
        consumer.synchronize()
        rig.pool.sync()
        want = expected_layer_rows(rig, h, 0)
        assert not same_rows(early, want), "a consumer that skips the wait was not caught"
        assert same_rows(consumer_rows(rig, 0, d2_t), want)
    finally:
        rig.close()


@pytest.mark.gpu
def test_failed_load_back_still_records_event():
    say("[events] failure injection")
    rig = Rig(SHAPE, seed=9)
    try:
        h, d, d2 = prepare(rig, 7)
        h_t, d2_t = cuda_i64(h), cuda_i64(d2)
        ev = B.HipEvent()
        with pytest.raises(B.HcError) as e:
            rig.pool.load_back_layer(SHAPE.layers, h_t, d2_t, ev)  # layer out of range
        assert e.value.code == B.HC_ERR_INVALID
        ev.synchronize()
        assert ev.query()
        ev2 = B.HipEvent()
        rc = B.lib.hc_load_back_layer(rig.pool.handle, 0, None, None, 5, ev2.handle)  # null lists
        assert rc == B.HC_ERR_INVALID
        ev2.synchronize()
        ev3 = B.HipEvent()
        rc = B.lib.hc_load_back_layer(None, 0, None, None, 5, ev3.handle)  # null pool: null stream
        assert rc == B.HC_ERR_INVALID
        ev3.synchronize()
        # the burst after a failed call is served normally
        dev0 = [[rig.dev[b][l].cpu().numpy() for l in range(SHAPE.layers)] for b in range(2)]
        for l in range(SHAPE.layers):
            rig.pool.load_back_layer(l, h_t, d2_t, None)
        rig.pool.sync()
        for l in range(SHAPE.layers):
            O.load_back_layer(rig.geom, l, dev0, rig.host.np, h, d2)
        for b in range(2):
            for l in range(SHAPE.layers):
                assert np.array_equal(rig.dev[b][l].cpu().numpy(), dev0[b][l])
    finally:
        rig.close()


@pytest.mark.gpu
def test_bad_indices_rejected_or_reported():
    say("[events] bad indices")
    rig = Rig(SHAPE, seed=10)
    try:
        h, d, d2 = prepare(rig, 9)
        host_before = rig.host.np.copy()
        # write-back: host list checked on the CPU before anything is enqueued
        bad_h = h.copy()
        bad_h[5] = SHAPE.host_pages * SHAPE.page_size
        with pytest.raises(B.HcError) as e:
            rig.pool.write_back_all_layers(cuda_i64(d), bad_h)
        assert e.value.code == B.HC_ERR_INVALID and "out of range" in str(e.value)
        dup = h.copy()
        dup[7] = dup[3]
        with pytest.raises(B.HcError):
            rig.pool.write_back_all_layers(cuda_i64(d), dup)
        rig.pool.sync()
        assert np.array_equal(rig.host.np, host_before)
        # load-back: device lists; the kernel skips the bad row and reports it
        bad_d = d2.copy()
        bad_d[3] = SHAPE.device_slots + 5
        dev0 = [[rig.dev[b][l].cpu().numpy() for l in range(SHAPE.layers)] for b in range(2)]
        rig.pool.load_back_layer(0, cuda_i64(h), cuda_i64(bad_d), None)
        with pytest.raises(B.HcError) as e:
            rig.pool.sync()
        assert e.value.code == B.HC_ERR_DEVICE and "first flagged list position 3)" in str(e.value), str(e.value)
        rig.pool.sync()  # the report is cleared once read
        keep = np.arange(h.size) != 3
        O.load_back_layer(rig.geom, 0, dev0, rig.host.np, h[keep], bad_d[keep])
        for b in range(2):
            assert np.array_equal(rig.dev[b][0].cpu().numpy(), dev0[b][0])
    finally:
        rig.close()


@pytest.mark.gpu
def test_validate_flag_reports_misaligned_page_blocks():
    say("[events] validate page blocks")
    rig = Rig(BLOCKS, seed=11, flags=B.HC_FLAG_VALIDATE)
    try:
        P = BLOCKS.page_size
        pages = W.host_pages(1, BLOCKS.host_pages, 4)
        h = W.whole_page_tokens(pages, P)
        d = W.page_aligned_slots(2, BLOCKS.device_slots, P, 4)
        d_bad = d.copy()
        d_bad[P:2 * P] += 1  # second page shifted off its boundary
        rig.pool.load_back_layer(0, cuda_i64(h), cuda_i64(d_bad), None)
        with pytest.raises(B.HcError) as e:
            rig.pool.sync()
        assert e.value.code == B.HC_ERR_DEVICE and "page-block" in str(e.value)
        assert f"first flagged list position {P})" in str(e.value), str(e.value)  # the shifted page's row 0
        rig.pool.load_back_layer(0, cuda_i64(h), cuda_i64(d), None)
        rig.pool.sync()
    finally:
        rig.close()


@pytest.mark.gpu
def test_negative_controls_corrupted_byte_and_skipped_layer():
    """The round-trip check catches a flipped host byte and a layer that was never
    loaded back, with exactly the oracle's count."""
    say("[controls] corrupted byte, skipped layer")
    rig = Rig(SHAPE, seed=13)
    try:
        h, d, d2 = prepare(rig, 11)
        # a flipped byte in one row of layer 2, sub-buffer 1
        off = int(O.host_offsets(rig.geom, 1, 2, h[5:6])[0]) + 17
        rig.host.np[off] ^= 0x5A
        skip = 4
        for l in range(SHAPE.layers):
            if l != skip:
                rig.pool.load_back_layer(l, cuda_i64(h), cuda_i64(d2), None)
        rig.pool.sync()
        got = rig.pool.round_trip_check(cuda_i64(d), cuda_i64(d2))
        dev = [[rig.dev[b][l].cpu().numpy() for l in range(SHAPE.layers)] for b in range(2)]
        want = O.round_trip_check(rig.geom, dev, d, d2)
        assert got == want
        assert want == 1 + 2 * h.size, "expected one corrupted row plus the skipped layer's rows"
    finally:
        rig.close()


@pytest.mark.gpu
def test_staged_write_back_with_poisoned_staging():
    """Staging filled with a poison byte before every burst: a copy that read staging
    before the gather wrote it would leave poison in the host pool."""
    from gpu_support import write_back_and_check
    say("[controls] poisoned staging")
    shape = W.PoolShape("poison_rows", 4, 16, ((T, 1024), (T, 512)), 16384, 128)
    rig = Rig(shape, seed=14, write_back_mode=B.HC_MODE_STAGED, staging_pages=6)
    try:
        for k in range(3):
            rig.staging.fill_(0xEE)
            torch.cuda.synchronize()
            pages = W.host_pages(20 + k, shape.host_pages, 40)
            h = W.whole_page_tokens(pages, shape.page_size)
            d = W.permutation_slots(30 + k, shape.device_slots, h.size)
            write_back_and_check(rig, d, h)
    finally:
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [B.HC_MODE_ZEROCOPY, B.HC_MODE_STAGED])
def test_validate_flag_reports_misaligned_page_blocks_on_write_back(mode):
    say(f"[events] validate page blocks on write-back, mode {mode}")
    rig = Rig(BLOCKS, seed=15, flags=B.HC_FLAG_VALIDATE, write_back_mode=mode, staging_pages=4)
    try:
        P = BLOCKS.page_size
        pages = W.host_pages(3, BLOCKS.host_pages, 4)
        h = W.whole_page_tokens(pages, P)
        d = W.page_aligned_slots(4, BLOCKS.device_slots, P, 4)
        rig.pool.write_back_all_layers(cuda_i64(d), h)
        rig.pool.sync()  # aligned: no report
        d_bad = d.copy()
        d_bad[2 * P:3 * P] -= 1  # third page off its boundary
        rig.pool.write_back_all_layers(cuda_i64(d_bad), h)
        with pytest.raises(B.HcError) as e:
            rig.pool.sync()
        assert e.value.code == B.HC_ERR_DEVICE and "page-block" in str(e.value)
        assert f"first flagged list position {2 * P})" in str(e.value), str(e.value)
    finally:
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [B.HC_MODE_ZEROCOPY, B.HC_MODE_STAGED], ids=["zerocopy", "staged"])
def test_done_event_covers_back_to_back_write_backs(mode):
    """Three write-back bursts enqueued back to back, no synchronization between them, over
    host pages that overlap from one burst to the next, each with a page named in part.
    Waiting on the last burst's done event alone (no stream or pool sync) must leave the
    whole host pool equal to the oracle's after all three in order: the event covers every
    copy and kernel of its burst, and a burst's host writes land after those of the burst
    before it (staged: the next burst's gathers into the shared staging chunk come after
    the copies that read it)."""
    say(f"[events] back-to-back write-backs, mode {mode}")
    shape = W.PoolShape("event_chain", 3, 16, ((T, 1024), (T, 512)), 16384, 96)
    rig = Rig(shape, seed=33, write_back_mode=mode, staging_pages=6 if mode == B.HC_MODE_STAGED else 0)
    try:
        dev0 = rig.dev_np()
        want = rig.host.np.copy()
        keep, events = [], []
        for k in range(3):
            pages = W.host_pages(40 + k, shape.host_pages, 40)
            h = W.whole_page_tokens(pages, shape.page_size)
            h = h[: h.size - 5]  # the last page named in part: zero-copy rows after the copies
            d = W.permutation_slots(50 + k, shape.device_slots, h.size)
            d_t = cuda_i64(d)
            ev = B.HipEvent()
            rig.pool.write_back_all_layers(d_t, h, ev)
            keep.append(d_t)
            events.append(ev)
            O.write_back(rig.geom, dev0, want, d, h)
        events[-1].synchronize()
        assert np.array_equal(rig.host.np, want), "host pool after the last burst's event differs from the oracle's"
        rig.pool.sync()
    finally:
        rig.close()


@pytest.mark.gpu
def test_block_pool_write_back_rejects_out_of_order_pages():
    """Whole pages whose rows are interleaved or out of order are refused on the CPU,
    before anything is enqueued: the kernels find a page's block at its row-0 position."""
    say("[events] page-block write-back, rows out of order")
    rig = Rig(BLOCKS, seed=16)
    try:
        P = BLOCKS.page_size
        pages = W.host_pages(5, BLOCKS.host_pages, 3)
        h = W.whole_page_tokens(pages, P)
        d = W.page_aligned_slots(6, BLOCKS.device_slots, P, 3)
        host_before = rig.host.np.copy()
        inter = np.concatenate([h[:P // 2], h[P:P + P // 2], h[P // 2:P], h[P + P // 2:2 * P], h[2 * P:]])
        for bad in (inter, np.concatenate([h[1:2], h[0:1], h[2:]])):
            with pytest.raises(B.HcError) as e:
                rig.pool.write_back_all_layers(cuda_i64(d), bad)
            assert e.value.code == B.HC_ERR_INVALID and "row order" in str(e.value)
        rig.pool.sync()
        assert np.array_equal(rig.host.np, host_before)
        write_back_and_check(rig, d, h)  # the same pages in order go through
    finally:
        rig.close()


def _raw(x):
    return B._V(x.ctypes.data if isinstance(x, np.ndarray) else x.data_ptr())


@pytest.mark.gpu
def test_index_lists_the_kernels_cannot_read_are_refused():
    """Lists in pageable host memory, or shorter than n, are refused before any launch (a
    kernel would fault on the first and read past the end of the second); the layer
    event is still recorded.  Pinned host lists are readable and move the same rows."""
    import ctypes
    say("[events] unreadable index lists refused")
    rig = Rig(SHAPE, seed=10)
    hip = B._hip
    short = ctypes.c_void_p()
    try:
        h, d, d2 = prepare(rig, 11)
        n = h.size
        h_t, d_t, d2_t = cuda_i64(h), cuda_i64(d), cuda_i64(d2)
        h_np = np.ascontiguousarray(h, dtype=np.int64)
        pool = rig.pool.handle

        def refused(rc, words):
            assert rc == B.HC_ERR_INVALID, rc
            msg = B.lib.hc_last_error().decode()
            assert all(w in msg for w in words), msg

        for l, (hh, dd, what) in enumerate([(h_np, d2_t, "host_idx"), (h_t, h_np, "device_idx")]):
            ev = B.HipEvent()
            refused(B.lib.hc_load_back_layer(pool, l, _raw(hh), _raw(dd), n, ev.handle), [what, "pageable"])
            ev.synchronize()  # recorded although nothing was launched
        refused(B.lib.hc_round_trip_check(pool, _raw(h_np), _raw(d_t), n, ctypes.byref(ctypes.c_int64())),
                ["idx_a", "pageable"])
        refused(B.lib.hc_write_back_all_layers(pool, _raw(d_t), _raw(h_t), n, None), ["host_idx", "host memory"])
        refused(B.lib.hc_write_back_all_layers(pool, _raw(h_np), _raw(h_np), n, None), ["device_idx", "pageable"])
        evs = (B._V * SHAPE.layers)(*[None] * SHAPE.layers)
        g = ctypes.c_void_p()
        refused(B.lib.hc_load_back_graph_create(pool, _raw(h_np), _raw(d2_t), n, evs, ctypes.byref(g)),
                ["host_idx", "pageable"])
        assert not g.value

        # a list shorter than n: an exact 4096-byte allocation holding 512 entries
        hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
        hip.hipMalloc.restype = ctypes.c_int
        assert hip.hipMalloc(ctypes.byref(short), 4096) == 0
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t),
                                              ctypes.c_void_p]
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), short) == 0
        assert base.value == short.value
        fits = size.value // 8
        assert fits < n
        refused(B.lib.hc_load_back_layer(pool, 0, short, _raw(d2_t), n, None), ["host_idx", "fewer than"])
        refused(B.lib.hc_round_trip_check(pool, _raw(d_t), short, n, ctypes.byref(ctypes.c_int64())),
                ["idx_b", "fewer than"])
        rig.pool.sync()  # nothing was flagged: no kernel ran

        # the binding refuses the wrong kinds before the library sees them
        with pytest.raises(TypeError):
            rig.pool.load_back_layer(0, torch.from_numpy(h_np), d2_t)
        with pytest.raises(TypeError):
            rig.pool.load_back_layer(0, h_t.to(torch.int32), d2_t)
        with pytest.raises(TypeError):
            rig.pool.write_back_all_layers(d_t, h_t)
        with pytest.raises(TypeError):
            rig.pool.round_trip_check(d_t[::2], d_t[1::2])

        # pinned host lists are readable by the kernels: the same rows land
        dev0 = rig.dev_np()
        pin_h = torch.from_numpy(h_np).pin_memory()
        pin_d = torch.from_numpy(np.ascontiguousarray(d2, dtype=np.int64)).pin_memory()
        for l in range(SHAPE.layers):
            assert B.lib.hc_load_back_layer(pool, l, _raw(pin_h), _raw(pin_d), n, None) == B.HC_OK
        rig.pool.sync()
        for l in range(SHAPE.layers):
            O.load_back_layer(rig.geom, l, dev0, rig.host.np, h, d2)
        for b in range(2):
            for l in range(SHAPE.layers):
                assert np.array_equal(rig.dev[b][l].cpu().numpy(), dev0[b][l])
    finally:
        if short.value:
            hip.hipFree.argtypes = [ctypes.c_void_p]
            hip.hipFree(short)
        rig.close()


@pytest.mark.gpu
def test_pool_buffers_smaller_than_the_layout_are_refused():
    """hc_pool_create checks that every device layer, the host pool and the staging
    chunk fit inside their allocations (a kernel would otherwise run past their ends)."""
    import ctypes
    say("[events] undersized pool buffers refused")
    hip = B._hip
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMalloc.restype = ctypes.c_int
    hip.hipFree.argtypes = [ctypes.c_void_p]
    L, P, E, S, H = 2, 16, 64, 1024, 8
    layer_bytes = S * E
    bufs = []

    def dmalloc(n):
        p = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(p), n) == 0
        bufs.append(p)
        return p.value

    probe, _k = B.make_desc(layers=L, page_size=P, subs=[(T, E, [1] * L)], device_slots=S, host_pages=H)
    host_need = B.host_pool_bytes(probe)
    host = B.HostBuffer(host_need)
    small_host = B.HostBuffer(host_need // 2)
    stream = torch.cuda.Stream()
    try:
        good = [dmalloc(layer_bytes) for _ in range(L)]
        img = B.staging_page_bytes(probe)

        def create(layers, host_ptr, staging_ptr=0, staging_bytes=0, mode=B.HC_MODE_ZEROCOPY):
            desc, keep = B.make_desc(layers=L, page_size=P, subs=[(T, E, layers)], device_slots=S, host_pages=H,
                                     host_ptr=host_ptr, host_bytes=host_need, staging_ptr=staging_ptr,
                                     staging_bytes=staging_bytes, stream_ptr=stream.cuda_stream,
                                     write_back_mode=mode)
            out = ctypes.c_void_p()
            rc = B.lib.hc_pool_create(ctypes.byref(desc), ctypes.byref(out))
            if rc == B.HC_OK:
                B.lib.hc_pool_destroy(out)
            return rc, B.lib.hc_last_error().decode()

        assert create(good, host.ptr.value)[0] == B.HC_OK
        rc, msg = create([good[0], dmalloc(layer_bytes - 4096)], host.ptr.value)
        assert rc == B.HC_ERR_INVALID and "sub-buffer 0 layer 1" in msg and "needed" in msg, msg
        rc, msg = create(good, small_host.ptr.value)
        assert rc == B.HC_ERR_INVALID and "host_base" in msg, msg
        staging = dmalloc(2 * img)
        assert create(good, host.ptr.value, staging, 2 * img, B.HC_MODE_STAGED)[0] == B.HC_OK
        rc, msg = create(good, host.ptr.value, staging, 4 * img, B.HC_MODE_STAGED)
        assert rc == B.HC_ERR_INVALID and "staging" in msg, msg
    finally:
        for p in bufs:
            hip.hipFree(p)
        small_host.free()
        host.free()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [B.HC_MODE_ZEROCOPY, B.HC_MODE_STAGED], ids=["zerocopy", "staged"])
def test_write_back_done_event(mode):
    """The write-back's event completes only after every host byte of the burst has landed
    (the host thread waits on the event alone, no pool sync), and it is recorded even when
    the call is refused."""
    say(f"[events] write-back done event, mode {mode}")
    rig = Rig(SHAPE, seed=17, write_back_mode=mode, staging_pages=3)
    try:
        pages = W.host_pages(18, SHAPE.host_pages, 11)
        h = W.whole_page_tokens(pages, SHAPE.page_size)
        h = np.concatenate([h, np.setdiff1d(np.arange(SHAPE.host_pages), pages)[0] * SHAPE.page_size + np.arange(5)])
        d = W.permutation_slots(19, SHAPE.device_slots, h.size)
        dev0, host0 = rig.dev_np(), rig.host.np.copy()
        torch.cuda.synchronize()
        done = B.HipEvent()
        rig.pool.write_back_all_layers(cuda_i64(d), h, done)
        done.synchronize()
        want = host0.copy()
        O.write_back(rig.geom, dev0, want, d, h)
        assert np.array_equal(rig.host.np, want), "host pool incomplete when the write-back event completed"
        refused = B.HipEvent()
        bad = h.copy()
        bad[2] = bad[1]  # a repeated host token: refused on the CPU
        with pytest.raises(B.HcError):
            rig.pool.write_back_all_layers(cuda_i64(d), bad, refused)
        refused.synchronize()
        assert refused.query()
        rig.pool.sync()
    finally:
        rig.close()
