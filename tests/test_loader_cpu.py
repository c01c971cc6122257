"""The asynchronous load-back enqueue, on the CPU.

The loader drives its device side through hc_loader_ops; these tests hand it
recording callbacks instead of HIP, then check the call sequence and the
threads that made each call -- the rules of the loader-thread page (sglang PR
38472, Modifications and Tests): inline mode keeps the plain sequence and starts
no thread; the async hand-over returns before the enqueue; a consumer waiting on
a layer blocks until that layer is recorded; a failed enqueue still completes
every layer and reports the error; bursts finish in submission order; reusing
the events of a queued burst waits for it; shutdown drains the queue."""
import ctypes
import threading
import time

import pytest

from host_device_page_amd import binding as B

L = 4
EV = [0x1000 + 16 * i for i in range(L)]
EV2 = [0x2000 + 16 * i for i in range(L)]


class Fake:
    """Records every device call with its thread; optional gates and failures."""

    def __init__(self):
        self.calls = []
        self.lock = threading.Lock()
        self.gates = {}     # (host_idx, layer) -> threading.Event the call waits on
        self.fail = {}      # (host_idx, layer) -> status to return
        self.ops = B.hc_loader_ops()
        self._fns = [B.LOAD_LAYER_FN(self._load), B.WAIT_EVENT_FN(self._wait), B.RECORD_EVENT_FN(self._record),
                     B.SYNC_EVENT_FN(self._sync), B.STREAM_WAIT_FN(self._stream_wait),
                     B.LAUNCH_GRAPH_FN(self._launch_graph)]
        (self.ops.load_layer, self.ops.wait_event, self.ops.record_event, self.ops.sync_event,
         self.ops.stream_wait, self.ops.launch_graph) = self._fns
        self.ops.ctx = None

    def _log(self, *c):
        with self.lock:
            self.calls.append((threading.get_ident(),) + c)

    def _load(self, ctx, layer, h, d, n, ev):
        gate = self.gates.get((h, layer))
        if gate is not None:
            assert gate.wait(10), "test gate never opened"
        self._log("load", layer, h, d, n, ev)
        return self.fail.get((h, layer), 0)

    def _wait(self, ctx, ev):
        self._log("wait_start", ev)
        return 0

    def _record(self, ctx, ev):
        self._log("record", ev)
        return 0

    def _sync(self, ctx, ev):
        self._log("sync", ev)
        return 0

    def _stream_wait(self, ctx, stream, ev):
        self._log("stream_wait", stream, ev)
        return 0

    def _launch_graph(self, ctx, graph):
        gate = self.gates.get(("graph", graph))
        if gate is not None:
            assert gate.wait(10), "test gate never opened"
        self._log("graph", graph)
        return self.fail.get(("graph", graph), 0)

    def seq(self):
        with self.lock:
            return [c[1:] for c in self.calls]

    def threads(self):
        with self.lock:
            return {c[0] for c in self.calls}


def test_inline_mode_keeps_the_plain_sequence_and_starts_no_thread():
    f = Fake()
    ld = B.Loader(None, L, asynchronous=False, ops=f.ops)
    assert ld.info() == (0, False)
    b = ld.submit(0x10, 0x20, 7, EV, start_event=0x99)
    assert b.query() == (L, True)
    assert f.seq() == [("wait_start", 0x99)] + [("load", l, 0x10, 0x20, 7, EV[l]) for l in range(L)]
    assert f.threads() == {threading.get_ident()}
    b.wait()
    b.release()
    ld.close()


def test_async_hand_over_returns_before_the_enqueue():
    f = Fake()
    f.gates[(0x10, 0)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    assert ld.info()[1] is True
    b = ld.submit(0x10, 0x20, 7, EV, start_event=0x99)
    time.sleep(0.05)
    assert b.query() == (0, False), "submit waited for the enqueue"
    f.gates[(0x10, 0)].set()
    ld.drain()
    assert b.query() == (L, True)
    seq = f.seq()
    assert seq[0] == ("wait_start", 0x99), "the start event must be waited on before the first layer"
    assert [c for c in seq if c[0] == "load"] == [("load", l, 0x10, 0x20, 7, EV[l]) for l in range(L)]
    assert threading.get_ident() not in f.threads(), "device calls must run on the loader thread"
    b.release()
    ld.close()


def test_consumer_blocks_until_the_layer_is_recorded():
    f = Fake()
    f.gates[(0x10, 2)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    b = ld.submit(0x10, 0x20, 7, EV)
    returned = threading.Event()

    def consumer():
        b.wait_layer(2, 0x77)
        returned.set()

    t = threading.Thread(target=consumer)
    t.start()
    time.sleep(0.1)
    assert not returned.is_set(), "a consumer passed a layer that was not recorded yet"
    b.wait_layer(1, 0x66)  # earlier layers are already available
    f.gates[(0x10, 2)].set()
    t.join(5)
    assert returned.is_set()
    seq = f.seq()
    assert seq.index(("stream_wait", 0x77, EV[2])) > seq.index(("load", 2, 0x10, 0x20, 7, EV[2]))
    b.release()
    ld.close()


def test_failed_enqueue_completes_every_layer_and_the_next_burst_is_served():
    f = Fake()
    f.fail[(0x10, 1)] = B.HC_ERR_HIP
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    b1 = ld.submit(0x10, 0x20, 7, EV)
    b2 = ld.submit(0x30, 0x40, 5, EV2)
    with pytest.raises(B.HcError) as e:
        b1.wait()
    assert e.value.code == B.HC_ERR_HIP
    b1.wait_layer(L - 1)  # released, not hung
    seq = f.seq()
    assert ("load", 1, 0x10, 0x20, 7, EV[1]) in seq
    assert ("load", 2, 0x10, 0x20, 7, EV[2]) not in seq, "layers after the failure were still enqueued"
    for l in (1, 2, 3):
        assert ("record", EV[l]) in seq, f"layer {l} event not completed after the failure"
    b2.wait()
    assert [c for c in f.seq() if c[0] == "load" and c[2] == 0x30] == \
        [("load", l, 0x30, 0x40, 5, EV2[l]) for l in range(L)]
    assert ld.info()[0] == 1
    b1.release()
    b2.release()
    ld.close()


def test_bursts_complete_in_submission_order():
    f = Fake()
    f.gates[(0x100, 0)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    evs = [[0x10000 * (k + 1) + 16 * l for l in range(L)] for k in range(3)]
    bursts = [ld.submit(0x100 * (k + 1), 0, 1, evs[k]) for k in range(3)]
    f.gates[(0x100, 0)].set()
    ld.drain()
    order = [c[2] for c in f.seq() if c[0] == "load"]
    assert order == [0x100] * L + [0x200] * L + [0x300] * L
    for b in bursts:
        b.release()
    ld.close()


def test_reusing_the_events_of_a_queued_burst_waits_for_it():
    f = Fake()
    gate = f.gates[(0x10, 0)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    b1 = ld.submit(0x10, 0x20, 7, EV)
    submitted = threading.Event()
    holder = {}

    def second():
        holder["b"] = ld.submit(0x30, 0x40, 5, EV)  # same events
        submitted.set()

    t = threading.Thread(target=second)
    t.start()
    time.sleep(0.1)
    assert not submitted.is_set(), "event reuse did not wait for the queued burst"
    gate.set()
    t.join(5)
    assert submitted.is_set()
    ld.drain()
    b1.release()
    holder["b"].release()
    ld.close()


def test_shutdown_drains_the_queue():
    f = Fake()
    gate = f.gates[(0x10, 3)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    b1 = ld.submit(0x10, 0, 1, EV)
    b2 = ld.submit(0x30, 0, 1, EV2)
    threading.Timer(0.1, gate.set).start()
    b1.release()
    b2.release()
    ld.close()
    loads = [c for c in f.seq() if c[0] == "load"]
    assert len(loads) == 2 * L


def test_argument_errors():
    f = Fake()
    out = ctypes.c_void_p()
    assert B.lib.hc_loader_create(None, None, L, 1, ctypes.byref(out)) == B.HC_ERR_INVALID
    assert B.lib.hc_loader_create(None, ctypes.byref(f.ops), 0, 1, ctypes.byref(out)) == B.HC_ERR_INVALID
    bad = B.hc_loader_ops()
    assert B.lib.hc_loader_create(None, ctypes.byref(bad), L, 1, ctypes.byref(out)) == B.HC_ERR_INVALID
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    with pytest.raises(B.HcError):
        ld.submit(0, 0, 1, [EV[0]] * L)  # repeated events
    with pytest.raises(B.HcError):
        ld.submit(0, 0, -1, EV)
    with pytest.raises(B.HcError):
        ld.submit(0, 0, 1, [EV[0], 0, EV[2], EV[3]])
    assert B.lib.hc_burst_wait_layer(None, 0, None) == B.HC_ERR_INVALID
    # the library reads exactly num_layers events: the binding refuses other counts
    for evs in (EV[:-1], EV + EV[:1]):
        with pytest.raises(ValueError):
            ld.submit(0, 0, 1, evs)
        with pytest.raises(ValueError):
            ld.submit_graph(1, evs)
    assert f.calls == []  # no refused submission reached the device ops
    ld.close()


def test_graph_bursts_share_the_fifo_and_flag_all_layers_at_once():
    f = Fake()
    gate = f.gates[("graph", 0x500)] = threading.Event()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    g1 = ld.submit_graph(0x500, EV, start_event=0x99)
    b2 = ld.submit(0x30, 0x40, 5, EV2)
    time.sleep(0.05)
    assert g1.query() == (0, False), "the graph burst was flagged before its launch"
    gate.set()
    g1.wait_layer(L - 1, 0x77)
    ld.drain()
    assert g1.query() == (L, True)
    seq = f.seq()
    assert seq[:2] == [("wait_start", 0x99), ("graph", 0x500)]
    assert [c for c in seq if c[0] == "load"] == [("load", l, 0x30, 0x40, 5, EV2[l]) for l in range(L)]
    assert seq.index(("graph", 0x500)) < seq.index(("load", 0, 0x30, 0x40, 5, EV2[0])), "FIFO order broken"
    assert ("stream_wait", 0x77, EV[L - 1]) in seq
    g1.release()
    b2.release()
    ld.close()


def test_failed_graph_launch_completes_every_layer():
    f = Fake()
    f.fail[("graph", 0x600)] = B.HC_ERR_HIP
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    g = ld.submit_graph(0x600, EV)
    with pytest.raises(B.HcError) as e:
        g.wait()
    assert e.value.code == B.HC_ERR_HIP
    for l in range(L):
        assert ("record", EV[l]) in f.seq(), f"layer {l} event not completed after the failed launch"
    assert ld.info()[0] == 1
    g.release()
    ld.close()


def test_graph_submit_needs_a_launch_op():
    f = Fake()
    f.ops.launch_graph = B.LAUNCH_GRAPH_FN()  # null
    ld = B.Loader(None, L, asynchronous=False, ops=f.ops)
    with pytest.raises(B.HcError) as e:
        ld.submit_graph(0x700, EV)
    assert e.value.code == B.HC_ERR_UNSUPPORTED
    out = ctypes.c_void_p()
    assert B.lib.hc_loader_submit_graph(None, None, None, None, ctypes.byref(out)) == B.HC_ERR_INVALID
    ld.close()


def test_destroy_refuses_while_a_burst_is_not_released():
    f = Fake()
    ld = B.Loader(None, L, asynchronous=True, ops=f.ops)
    b = ld.submit(0x10, 0, 1, EV)
    b.wait()
    assert B.lib.hc_loader_destroy(ld.handle) == B.HC_ERR_INVALID
    assert "not released" in B.lib.hc_last_error().decode()
    b.release()
    ld.close()  # now it goes
    assert not ld.handle.value
