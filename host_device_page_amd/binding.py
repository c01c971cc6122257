"""ctypes binding of libhc.so -- argument marshalling only.

Every function here forwards to the C ABI declared in ``include/hc.h`` under
the same name.  Torch supplies device memory and streams; the pinned host pool
comes from ``hc_host_alloc``.  Importing this module fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import weakref

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# HC_LIBRARY points the binding at another build of the same sources (tuning variants).
LIB_PATH = os.environ.get("HC_LIBRARY") or os.path.join(_PKG, "libhc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m host_device_page_amd.build` "
                      "(hipcc, gfx950); the transfer path has no fallback")

lib = ctypes.CDLL(LIB_PATH)

HC_OK = 0
HC_ERR_INVALID = -1
HC_ERR_UNSUPPORTED = -2
HC_ERR_HIP = -3
HC_ERR_NOMEM = -4
HC_ERR_DEVICE = -5
HC_ERR_BUSY = -6
HC_H2H_DUMP = 0
HC_H2H_LOAD = 1
HC_TOKEN_ROWS = 0
HC_PAGE_BLOCKS = 1
HC_LAYOUT_PAGE_FIRST = 0
HC_LAYOUT_KV_SPLIT_SHARD = 1
HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR = 2
HC_MODE_AUTO = 0
HC_MODE_STAGED = 1
HC_MODE_ZEROCOPY = 2
HC_FLAG_VALIDATE = 1
HC_FLAG_PROFILE = 2
HC_MAX_SUBBUFS = 4
HC_DUPLEX_LOAD_BACK_CTAS = 8
HC_NOALLOC_MAX_TOKENS = 262144

# hc_pool_kernel_time kinds
KIND_GATHER, KIND_ZC_WRITE, KIND_ZC_READ, KIND_PADS, KIND_COMPARE, KIND_COPY_ENGINE, KIND_PACK, KIND_UNPACK = range(8)


class hc_subbuf_desc(ctypes.Structure):
    _fields_ = [("granularity", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int64), ("device_layers", ctypes.POINTER(ctypes.c_void_p))]


class hc_pool_desc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_subbufs", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("sub", hc_subbuf_desc * HC_MAX_SUBBUFS),
                ("device_slots", ctypes.c_int64), ("host_pages", ctypes.c_int64),
                ("shard_align", ctypes.c_int64),
                ("host_base", ctypes.c_void_p), ("host_bytes", ctypes.c_int64),
                ("staging", ctypes.c_void_p), ("staging_bytes", ctypes.c_int64),
                ("copy_stream", ctypes.c_void_p),
                ("write_back_mode", ctypes.c_int32), ("load_back_mode", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("max_ctas", ctypes.c_int32)]


class hc_pool_stats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "write_back_calls", "write_back_tokens", "write_back_bytes",
        "load_back_calls", "load_back_tokens", "load_back_bytes", "device_errors")]


_D = ctypes.POINTER(hc_pool_desc)
_V = ctypes.c_void_p

LOAD_LAYER_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, ctypes.c_int32, _V, _V, ctypes.c_int64, _V)
WAIT_EVENT_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, _V)
RECORD_EVENT_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, _V)
SYNC_EVENT_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, _V)
STREAM_WAIT_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, _V, _V)
LAUNCH_GRAPH_FN = ctypes.CFUNCTYPE(ctypes.c_int, _V, _V)


class hc_loader_ops(ctypes.Structure):
    _fields_ = [("ctx", _V), ("load_layer", LOAD_LAYER_FN), ("wait_event", WAIT_EVENT_FN),
                ("record_event", RECORD_EVENT_FN), ("sync_event", SYNC_EVENT_FN),
                ("stream_wait", STREAM_WAIT_FN), ("launch_graph", LAUNCH_GRAPH_FN)]
_I64P = ctypes.POINTER(ctypes.c_int64)
_SIGS = {
    "hc_desc_check": (ctypes.c_int, [_D]),
    "hc_host_pool_bytes": (ctypes.c_int, [_D, _I64P]),
    "hc_staging_page_bytes": (ctypes.c_int, [_D, _I64P]),
    "hc_host_offset": (ctypes.c_int, [_D, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _I64P]),
    "hc_host_alloc": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_V)]),
    "hc_host_free": (ctypes.c_int, [_V]),
    "hc_pool_create": (ctypes.c_int, [_D, ctypes.POINTER(_V)]),
    "hc_pool_destroy": (ctypes.c_int, [_V]),
    "hc_pool_mode": (ctypes.c_int, [_V, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "hc_pool_sync": (ctypes.c_int, [_V]),
    "hc_write_back_all_layers": (ctypes.c_int, [_V, _V, _V, ctypes.c_int64, _V]),
    "hc_write_back_all_layers_noalloc": (ctypes.c_int, [_V, _V, _V, ctypes.c_int64, _V]),
    "hc_load_back_layer": (ctypes.c_int, [_V, ctypes.c_int32, _V, _V, ctypes.c_int64, _V]),
    "hc_round_trip_check": (ctypes.c_int, [_V, _V, _V, ctypes.c_int64, _I64P]),
    "hc_layer_pack_bytes": (ctypes.c_int, [_V, ctypes.c_int64, _I64P]),
    "hc_layer_pack": (ctypes.c_int, [_V, ctypes.c_int32, _V, ctypes.c_int64, _V, ctypes.c_int64, _V]),
    "hc_layer_unpack": (ctypes.c_int, [_V, ctypes.c_int32, _V, ctypes.c_int64, _V, ctypes.c_int64, _V]),
    "hc_load_back_graph_create": (ctypes.c_int, [_V, _V, _V, ctypes.c_int64, ctypes.POINTER(_V),
                                                 ctypes.POINTER(_V)]),
    "hc_load_back_graph_launch": (ctypes.c_int, [_V]),
    "hc_load_back_graph_destroy": (ctypes.c_int, [_V]),
    "hc_pool_kernel_time": (ctypes.c_int, [_V, ctypes.c_int32, ctypes.c_int32, _I64P,
                                           ctypes.POINTER(ctypes.c_double)]),
    "hc_pool_get_stats": (ctypes.c_int, [_V, ctypes.POINTER(hc_pool_stats)]),
    "hc_loader_create": (ctypes.c_int, [_V, ctypes.POINTER(hc_loader_ops), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(_V)]),
    "hc_loader_submit": (ctypes.c_int, [_V, _V, _V, ctypes.c_int64, ctypes.POINTER(_V), _V, ctypes.POINTER(_V)]),
    "hc_loader_submit_graph": (ctypes.c_int, [_V, _V, ctypes.POINTER(_V), _V, ctypes.POINTER(_V)]),
    "hc_burst_wait_layer": (ctypes.c_int, [_V, ctypes.c_int32, _V]),
    "hc_burst_wait": (ctypes.c_int, [_V]),
    "hc_burst_query": (ctypes.c_int, [_V, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "hc_burst_release": (ctypes.c_int, [_V]),
    "hc_loader_drain": (ctypes.c_int, [_V]),
    "hc_loader_info": (ctypes.c_int, [_V, _I64P, ctypes.POINTER(ctypes.c_int32)]),
    "hc_loader_destroy": (ctypes.c_int, [_V]),
    "hc_h2h_create": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(_V)]),
    "hc_h2h_submit": (ctypes.c_int, [_V, ctypes.c_int32, ctypes.c_int32, _I64P, ctypes.POINTER(_V),
                                     ctypes.POINTER(_V), ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_V)]),
    "hc_h2h_wait": (ctypes.c_int, [_V]),
    "hc_h2h_release": (ctypes.c_int, [_V]),
    "hc_h2h_outstanding": (ctypes.c_int, [_V, _I64P, _I64P]),
    "hc_h2h_destroy": (ctypes.c_int, [_V]),
    "hc_cache_fingerprint": (ctypes.c_int, [_D, ctypes.c_char_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]),
    "hc_last_error": (ctypes.c_char_p, []),
    "hc_version": (ctypes.c_int, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class HcError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib.hc_last_error().decode(errors="replace")
        super().__init__(f"{where}: status {code}: {msg}")


def check(code: int, where: str) -> None:
    if code != HC_OK:
        raise HcError(code, where)


# ---------------------------------------------------------------- HIP events (plumbing)
_hip = ctypes.CDLL("libamdhip64.so")
for _name, _args in {"hipEventCreateWithFlags": [ctypes.POINTER(_V), ctypes.c_uint],
                     "hipEventDestroy": [_V], "hipEventSynchronize": [_V], "hipEventQuery": [_V],
                     "hipEventRecord": [_V, _V], "hipStreamWaitEvent": [_V, _V, ctypes.c_uint],
                     "hipEventElapsedTime": [ctypes.POINTER(ctypes.c_float), _V, _V],
                     "hipMemsetAsync": [_V, ctypes.c_int, ctypes.c_size_t, _V],
                     "hipStreamSynchronize": [_V]}.items():
    getattr(_hip, _name).argtypes = _args
    getattr(_hip, _name).restype = ctypes.c_int


def _hip_check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what} failed with hipError {code}")


class HipEvent:
    """A raw hipEvent_t (the layer-done events handed to hc_load_back_layer)."""

    def __init__(self, timing: bool = False):
        self.handle = _V()
        _hip_check(_hip.hipEventCreateWithFlags(ctypes.byref(self.handle), 0 if timing else 2),
                   "hipEventCreateWithFlags")

    def wait_on(self, stream) -> None:
        """Make `stream` (a torch stream) wait for this event."""
        _hip_check(_hip.hipStreamWaitEvent(_V(stream.cuda_stream), self.handle, 0), "hipStreamWaitEvent")

    def record(self, stream) -> None:
        _hip_check(_hip.hipEventRecord(self.handle, _V(stream.cuda_stream)), "hipEventRecord")

    def synchronize(self) -> None:
        _hip_check(_hip.hipEventSynchronize(self.handle), "hipEventSynchronize")

    def query(self) -> bool:
        return _hip.hipEventQuery(self.handle) == 0

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        _hip_check(_hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle), "hipEventElapsedTime")
        return float(ms.value)

    def destroy(self) -> None:
        if getattr(self, "handle", None) and self.handle.value:
            _hip.hipEventDestroy(self.handle)
            self.handle = _V()

    def __del__(self):
        try:
            self.destroy()
        except Exception:  # interpreter shutdown: the HIP module may already be gone
            pass


class LoadBackGraph:
    """hc_lb_graph: a captured per-layer load-back burst; launch() enqueues one replay
    on the pool's copy stream.  Keeps the index tensors and events alive."""

    def __init__(self, pool, host_idx, device_idx, events):
        n = _index_list(device_idx, "device_idx", True)
        if _index_list(host_idx, "host_idx", True) != n:
            raise ValueError("host_idx and device_idx differ in length")
        if len(events) != pool.layers:
            raise ValueError(f"{len(events)} layer events for a pool of {pool.layers} layers")
        arr = (_V * len(events))(*[e.handle.value if e is not None else None for e in events])
        self._refs = (pool, host_idx, device_idx, list(events), arr)
        self.handle = _V()
        check(lib.hc_load_back_graph_create(pool.handle, _V(_ptr(host_idx)), _V(_ptr(device_idx)), n, arr,
                                            ctypes.byref(self.handle)), "hc_load_back_graph_create")

    def launch(self) -> None:
        check(lib.hc_load_back_graph_launch(self.handle), "hc_load_back_graph_launch")

    def close(self) -> None:
        if self.handle.value:
            check(lib.hc_load_back_graph_destroy(self.handle), "hc_load_back_graph_destroy")
            self.handle = _V()
            # replays already enqueued still read the lists
            _in_use_on(self._refs[0].stream, self._refs[1], self._refs[2])

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- pinned host memory
class HostBuffer:
    """Pinned host memory from hc_host_alloc; .np is a uint8 numpy view of it."""

    def __init__(self, nbytes: int, noncoherent: bool = False):
        self.nbytes = int(nbytes)
        self.ptr = _V()
        check(lib.hc_host_alloc(self.nbytes, 1 if noncoherent else 0, ctypes.byref(self.ptr)), "hc_host_alloc")
        self.np = np.ctypeslib.as_array((ctypes.c_uint8 * self.nbytes).from_address(self.ptr.value))

    def fill(self, byte: int, stream=None) -> None:
        """Fill every byte through the device mapping (a HIP memset; plumbing for tests)."""
        s = _V(stream.cuda_stream) if stream is not None else _V()
        _hip_check(_hip.hipMemsetAsync(self.ptr, int(byte), self.nbytes, s), "hipMemsetAsync")
        _hip_check(_hip.hipStreamSynchronize(s), "hipStreamSynchronize")

    def free(self) -> None:
        if self.ptr.value:
            self.np = None
            check(lib.hc_host_free(self.ptr), "hc_host_free")
            self.ptr = _V()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ---------------------------------------------------------------- descriptors and pools
def make_desc(*, layers: int, page_size: int, subs, device_slots: int, host_pages: int,
              layout: int = HC_LAYOUT_PAGE_FIRST, shard_align: int = 4096, host_ptr: int = 0,
              host_bytes: int = 0, staging_ptr: int = 0, staging_bytes: int = 0, stream_ptr: int = 0,
              write_back_mode: int = HC_MODE_AUTO, load_back_mode: int = HC_MODE_AUTO, flags: int = 0,
              max_ctas: int = 0):
    """Build an hc_pool_desc.  subs: [(granularity, elem_bytes, [layer device pointers])].
    Returns (desc, keepalive) -- keep the second value alive as long as desc is used."""
    d = hc_pool_desc()
    d.num_layers, d.page_size, d.num_subbufs, d.layout = layers, page_size, len(subs), layout
    keep = []
    for b, (gran, elem, ptrs) in enumerate(subs):
        arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])
        keep.append(arr)
        d.sub[b].granularity = gran
        d.sub[b].reserved = 0
        d.sub[b].elem_bytes = elem
        d.sub[b].device_layers = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    d.device_slots, d.host_pages, d.shard_align = device_slots, host_pages, shard_align
    d.host_base, d.host_bytes = host_ptr or None, host_bytes
    d.staging, d.staging_bytes = staging_ptr or None, staging_bytes
    d.copy_stream = stream_ptr or None
    d.write_back_mode, d.load_back_mode, d.flags, d.max_ctas = write_back_mode, load_back_mode, flags, max_ctas
    return d, keep


def host_pool_bytes(desc) -> int:
    out = ctypes.c_int64()
    check(lib.hc_host_pool_bytes(ctypes.byref(desc), ctypes.byref(out)), "hc_host_pool_bytes")
    return out.value


def staging_page_bytes(desc) -> int:
    out = ctypes.c_int64()
    check(lib.hc_staging_page_bytes(ctypes.byref(desc), ctypes.byref(out)), "hc_staging_page_bytes")
    return out.value


def host_offset(desc, sub: int, page: int, layer: int, row: int) -> int:
    out = ctypes.c_int64()
    check(lib.hc_host_offset(ctypes.byref(desc), sub, page, layer, row, ctypes.byref(out)), "hc_host_offset")
    return out.value


def _staging_bytes(x, what: str) -> int:
    """Size in bytes of an exchange staging buffer: a contiguous CUDA tensor."""
    if not getattr(x, "is_cuda", False) or not x.is_contiguous():
        raise TypeError(f"{what} must be a contiguous CUDA tensor")
    return x.numel() * x.element_size()


def _ptr(x) -> int:
    """Address of a torch tensor, a numpy array, a HostBuffer or an int."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, HostBuffer):
        return x.ptr.value
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _index_list(x, what: str, on_device: bool):
    """Check an index list argument and return its element count.  torch tensors and numpy
    arrays must be int64 and contiguous; device lists must be CUDA tensors, the
    write-back's host list must not be one (the library rechecks the memory itself)."""
    if isinstance(x, np.ndarray):
        if on_device:
            raise TypeError(f"{what} must be an int64 CUDA tensor, not a numpy array")
        if x.dtype != np.int64 or not x.flags.c_contiguous:
            raise TypeError(f"{what} must be a C-contiguous int64 array")
        return int(x.size)
    if hasattr(x, "is_cuda"):
        if x.dtype != _torch_int64() or not x.is_contiguous():
            raise TypeError(f"{what} must be a contiguous int64 tensor")
        if x.is_cuda != on_device:
            raise TypeError(f"{what} must be a {'CUDA' if on_device else 'CPU'} tensor")
        return int(x.numel())
    raise TypeError(f"{what}: expected a torch tensor or numpy array")


def _in_use_on(stream, *tensors):
    """The library reads these device tensors on `stream` after the call returns: tell
    torch's caching allocator, so a tensor freed meanwhile (a temporary argument) is not
    handed to another allocation before that stream's work is done."""
    if stream is None or not hasattr(stream, "cuda_stream"):
        return
    for t in tensors:
        if getattr(t, "is_cuda", False):
            t.record_stream(stream)


def _torch_int64():
    import torch
    return torch.int64


class Pool:
    """Owns one hc_pool handle.  device_layers[b][l] are torch CUDA tensors (or raw
    addresses); host is a HostBuffer (None with host_pages=0: a device-only pool for the
    layer exchange); staging a torch CUDA tensor or None; stream a torch.cuda.Stream
    (the copy stream)."""

    def __init__(self, *, layers, page_size, subs, device_slots, host_pages, device_layers, host,
                 stream, layout=HC_LAYOUT_PAGE_FIRST, shard_align=4096, staging=None,
                 write_back_mode=HC_MODE_AUTO, load_back_mode=HC_MODE_AUTO, flags=0, max_ctas=0):
        sub_specs = [(g, e, [_ptr(t) for t in device_layers[b]]) for b, (g, e) in enumerate(subs)]
        self.stream = stream
        self.layers = layers
        self.desc, self._keep = make_desc(
            layers=layers, page_size=page_size, subs=sub_specs, device_slots=device_slots,
            host_pages=host_pages, layout=layout, shard_align=shard_align, host_ptr=_ptr(host),
            host_bytes=host.nbytes if host is not None else 0, staging_ptr=_ptr(staging),
            staging_bytes=(staging.numel() * staging.element_size()) if staging is not None else 0,
            stream_ptr=stream.cuda_stream if stream is not None else 0,
            write_back_mode=write_back_mode, load_back_mode=load_back_mode, flags=flags, max_ctas=max_ctas)
        self._refs = (device_layers, host, staging)
        self._args = dict(layers=layers, page_size=page_size, subs=subs, device_slots=device_slots,
                          host_pages=host_pages, device_layers=device_layers, host=host, layout=layout,
                          shard_align=shard_align, load_back_mode=load_back_mode, flags=flags)
        self.handle = _V()
        check(lib.hc_pool_create(ctypes.byref(self.desc), ctypes.byref(self.handle)), "hc_pool_create")

    def sibling(self, stream, *, max_ctas: int = 0, write_back_mode: int = HC_MODE_ZEROCOPY,
                staging=None) -> "Pool":
        """Another pool over the same device and host buffers, on its own copy stream, with
        its own grid cap, write-back mode and staging: a write-back and a load-back can then
        run at the same time (their rows must not overlap).  Beside a staged write-back, a
        sibling with max_ctas=8 that loads back moves both directions near 45 GB/s each;
        at the default 16 the load-back keeps its full rate and the write-back backs off."""
        return Pool(stream=stream, staging=staging, write_back_mode=write_back_mode, max_ctas=max_ctas,
                    **self._args)

    def duplex_partner(self, stream) -> "Pool":
        """The load-back pool to run beside this staged write-back pool: a zero-copy sibling
        on `stream` capped at HC_DUPLEX_LOAD_BACK_CTAS workgroups, the pairing that moves
        the most bytes in both directions at once (both near 45 GB/s, measured).  Keep the
        default sibling (16 workgroups) when the load-back must keep its full rate."""
        if self.mode(0) != HC_MODE_STAGED:
            raise ValueError("duplex_partner pairs with a staged write-back pool: a zero-copy write-back "
                             "starves concurrent load-backs")
        return self.sibling(stream, max_ctas=HC_DUPLEX_LOAD_BACK_CTAS)

    def mode(self, which: int) -> int:
        out = ctypes.c_int32()
        check(lib.hc_pool_mode(self.handle, which, ctypes.byref(out)), "hc_pool_mode")
        return out.value

    def write_back_all_layers(self, device_idx, host_idx, event: HipEvent | None = None) -> None:
        """device_idx: int64 CUDA tensor; host_idx: int64 CPU tensor or numpy array."""
        n = _index_list(device_idx, "device_idx", True)
        if _index_list(host_idx, "host_idx", False) != n:
            raise ValueError("host_idx and device_idx differ in length")
        rc = lib.hc_write_back_all_layers(self.handle, _V(_ptr(device_idx)), _V(_ptr(host_idx)), n,
                                          event.handle if event else None)
        _in_use_on(self.stream, device_idx)  # also after a failure that enqueued part of the burst
        check(rc, "hc_write_back_all_layers")

    def write_back_all_layers_noalloc(self, device_idx, host_idx: "HostBuffer", n: int,
                                      event: HipEvent | None = None) -> None:
        """The write-back that allocates nothing (zero-copy pools): device_idx an int64 CUDA
        tensor, host_idx a HostBuffer whose first n int64 entries are the host tokens."""
        if _index_list(device_idx, "device_idx", True) != n:
            raise ValueError("device_idx must hold n entries")
        if not isinstance(host_idx, HostBuffer) or host_idx.nbytes < 8 * n:
            raise TypeError("host_idx must be a HostBuffer of at least n int64 entries")
        rc = lib.hc_write_back_all_layers_noalloc(self.handle, _V(_ptr(device_idx)), _V(_ptr(host_idx)), n,
                                                  event.handle if event else None)
        _in_use_on(self.stream, device_idx)
        check(rc, "hc_write_back_all_layers_noalloc")

    def load_back_layer(self, layer: int, host_idx, device_idx, event: HipEvent | None = None) -> None:
        """host_idx, device_idx: int64 CUDA tensors."""
        n = _index_list(device_idx, "device_idx", True)
        if _index_list(host_idx, "host_idx", True) != n:
            raise ValueError("host_idx and device_idx differ in length")
        rc = lib.hc_load_back_layer(self.handle, layer, _V(_ptr(host_idx)), _V(_ptr(device_idx)), n,
                                    event.handle if event else None)
        _in_use_on(self.stream, host_idx, device_idx)
        check(rc, "hc_load_back_layer")

    # The host-pool method names the pages use (hybrid-pool write-back page, host-pool
    # excerpt; loader-thread page, Motivation), in their argument order, host indices
    # first.  The device pool is this pool's own device side, so it is no argument.
    def backup_from_device_all_layer(self, host_indices, device_indices, event: HipEvent | None = None) -> None:
        self.write_back_all_layers(device_indices, host_indices, event)

    def load_to_device_per_layer(self, host_indices, device_indices, layer_id: int,
                                 event: HipEvent | None = None) -> None:
        self.load_back_layer(layer_id, host_indices, device_indices, event)

    def capture_load_back(self, host_idx, device_idx, events) -> "LoadBackGraph":
        """Capture the per-layer load-back of (host_idx, device_idx) with one event per
        layer (None entries: no record) into a replayable graph."""
        return LoadBackGraph(self, host_idx, device_idx, events)

    def round_trip_check(self, idx_a, idx_b) -> int:
        out = ctypes.c_int64()
        n = _index_list(idx_a, "idx_a", True)
        if _index_list(idx_b, "idx_b", True) != n:
            raise ValueError("idx_a and idx_b differ in length")
        check(lib.hc_round_trip_check(self.handle, _V(_ptr(idx_a)), _V(_ptr(idx_b)), n, ctypes.byref(out)),
              "hc_round_trip_check")
        return out.value

    # Layer exchange of a rank-sharded host tier (rank-sharded tier page, Modifications):
    # the owner packs a loaded layer's rows, the other ranks unpack the broadcast bytes.
    def layer_pack_bytes(self, n: int) -> int:
        out = ctypes.c_int64()
        check(lib.hc_layer_pack_bytes(self.handle, n, ctypes.byref(out)), "hc_layer_pack_bytes")
        return out.value

    def layer_pack(self, layer: int, device_idx, dst, event: HipEvent | None = None) -> None:
        """dst <- rows of `layer` at device_idx, sub-buffer after sub-buffer (dst: CUDA tensor)."""
        n = _index_list(device_idx, "device_idx", True)
        rc = lib.hc_layer_pack(self.handle, layer, _V(_ptr(device_idx)), n, _V(_ptr(dst)), _staging_bytes(dst, "dst"),
                               event.handle if event else None)
        _in_use_on(self.stream, device_idx, dst)
        check(rc, "hc_layer_pack")

    def layer_unpack(self, layer: int, src, device_idx, event: HipEvent | None = None) -> None:
        """Rows of `layer` at device_idx <- src, in the order layer_pack writes."""
        n = _index_list(device_idx, "device_idx", True)
        rc = lib.hc_layer_unpack(self.handle, layer, _V(_ptr(src)), _staging_bytes(src, "src"), _V(_ptr(device_idx)), n,
                                 event.handle if event else None)
        _in_use_on(self.stream, device_idx, src)
        check(rc, "hc_layer_unpack")

    def sync(self) -> None:
        check(lib.hc_pool_sync(self.handle), "hc_pool_sync")

    def stats(self) -> dict:
        """Running totals of the pool's enqueued transfer calls (hc_pool_get_stats)."""
        out = hc_pool_stats()
        check(lib.hc_pool_get_stats(self.handle, ctypes.byref(out)), "hc_pool_get_stats")
        return {name: getattr(out, name) for name, _ in hc_pool_stats._fields_}

    def kernel_time(self, kind: int, reset: bool = False):
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        check(lib.hc_pool_kernel_time(self.handle, kind, 1 if reset else 0, ctypes.byref(n), ctypes.byref(ms)),
              "hc_pool_kernel_time")
        return n.value, ms.value

    def close(self) -> None:
        if self.handle.value:
            check(lib.hc_pool_destroy(self.handle), "hc_pool_destroy")
            self.handle = _V()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- asynchronous load-back enqueue
class Burst:
    """One submitted load-back burst (hc_burst)."""

    def __init__(self, handle, keep, loader):
        self.handle = handle
        self._keep = keep  # index tensors and event array stay alive until release
        self._loader = loader  # a burst must be released before its loader is destroyed

    def wait_layer(self, layer: int, consumer_stream=None) -> None:
        """consumer_stream: a torch stream, a raw address (int), or None (block the thread)."""
        s = consumer_stream
        if s is not None and not isinstance(s, int):
            s = s.cuda_stream
        check(lib.hc_burst_wait_layer(self.handle, layer, _V(s) if s else None), "hc_burst_wait_layer")

    def wait(self) -> None:
        check(lib.hc_burst_wait(self.handle), "hc_burst_wait")

    def status(self) -> int:
        return lib.hc_burst_wait(self.handle)

    def query(self):
        n, done = ctypes.c_int32(), ctypes.c_int32()
        check(lib.hc_burst_query(self.handle, ctypes.byref(n), ctypes.byref(done)), "hc_burst_query")
        return n.value, bool(done.value)

    def release(self) -> None:
        if self.handle.value:
            check(lib.hc_burst_release(self.handle), "hc_burst_release")
            self.handle = _V()
            self._keep = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


class Loader:
    """hc_loader: per-layer load-back bursts enqueued by a worker thread (async) or inline.
    pool: a Pool (device operations of that pool) or None with explicit ops."""

    def __init__(self, pool: "Pool | None", num_layers: int, asynchronous: bool = True, ops: hc_loader_ops = None):
        self.handle = _V()
        self._pool = pool
        self._ops = ops
        self._bursts = weakref.WeakSet()
        check(lib.hc_loader_create(pool.handle if pool is not None else None,
                                   ctypes.byref(ops) if ops is not None else None,
                                   num_layers, 1 if asynchronous else 0, ctypes.byref(self.handle)),
              "hc_loader_create")
        self.num_layers = num_layers

    def _event_array(self, layer_events):
        # the library reads exactly num_layers entries
        if len(layer_events) != self.num_layers:
            raise ValueError(f"{len(layer_events)} layer events for a loader of {self.num_layers} layers")
        raw = [e.handle.value if isinstance(e, HipEvent) else int(e) for e in layer_events]
        return (_V * len(raw))(*raw)

    def submit(self, host_idx, device_idx, n: int, layer_events, start_event=None) -> Burst:
        """layer_events: HipEvent objects or raw handles (ints); start_event likewise or None."""
        arr = self._event_array(layer_events)
        st = start_event.handle.value if isinstance(start_event, HipEvent) else start_event
        out = _V()
        check(lib.hc_loader_submit(self.handle, _V(_ptr(host_idx)), _V(_ptr(device_idx)), n, arr,
                                   _V(st) if st else None, ctypes.byref(out)), "hc_loader_submit")
        if self._pool is not None:  # the worker enqueues on the pool's stream, maybe after the burst is released
            _in_use_on(self._pool.stream, host_idx, device_idx)
        b = Burst(out, (host_idx, device_idx, arr, layer_events, start_event), self)
        self._bursts.add(b)
        return b

    def submit_graph(self, graph, layer_events, start_event=None) -> Burst:
        """graph: a LoadBackGraph of this loader's pool (or a raw handle for custom ops);
        layer_events: the events it was captured with, in layer order."""
        arr = self._event_array(layer_events)
        st = start_event.handle.value if isinstance(start_event, HipEvent) else start_event
        gh = graph.handle if isinstance(graph, LoadBackGraph) else _V(graph)
        out = _V()
        check(lib.hc_loader_submit_graph(self.handle, gh, arr, _V(st) if st else None, ctypes.byref(out)),
              "hc_loader_submit_graph")
        b = Burst(out, (graph, arr, layer_events, start_event), self)
        self._bursts.add(b)
        return b

    def drain(self) -> None:
        check(lib.hc_loader_drain(self.handle), "hc_loader_drain")

    def info(self):
        f, r = ctypes.c_int64(), ctypes.c_int32()
        check(lib.hc_loader_info(self.handle, ctypes.byref(f), ctypes.byref(r)), "hc_loader_info")
        return f.value, bool(r.value)

    def close(self) -> None:
        if self.handle.value:
            check(lib.hc_loader_drain(self.handle), "hc_loader_drain")
            for b in list(self._bursts):
                b.release()
            check(lib.hc_loader_destroy(self.handle), "hc_loader_destroy")
            self.handle = _V()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- host-to-host shard copies
class H2H:
    """hc_h2h: CPU copy workers moving host pages to / from store shards."""

    def __init__(self, workers: int = 4, queue_depth: int = 1024):
        self.handle = _V()
        self._live = {}  # request handle -> the address arrays it was submitted with
        check(lib.hc_h2h_create(workers, queue_depth, ctypes.byref(self.handle)), "hc_h2h_create")

    def submit(self, direction: int, tensor_bytes, tensor_pages, shards, shard_bytes: int):
        """tensor_pages: [n][tensors] addresses; shards: [n] addresses.  Returns a request handle."""
        T = len(tensor_bytes)
        n = len(shards)
        sizes = (ctypes.c_int64 * T)(*tensor_bytes)
        pages = (_V * max(1, n * T))(*[int(a) for row in tensor_pages for a in row])
        sh = (_V * max(1, n))(*[int(a) for a in shards])
        out = _V()
        check(lib.hc_h2h_submit(self.handle, direction, T, sizes, pages, sh, shard_bytes, n, ctypes.byref(out)),
              "hc_h2h_submit")
        self._live[out.value] = (sizes, pages, sh)
        return out

    def wait(self, req) -> None:
        """Waits for the request's shards, then releases it."""
        self._live.pop(req.value, None)
        check(lib.hc_h2h_release(req), "hc_h2h_release")

    def outstanding(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        check(lib.hc_h2h_outstanding(self.handle, ctypes.byref(a), ctypes.byref(b)), "hc_h2h_outstanding")
        return a.value, b.value

    def close(self) -> None:
        if self.handle.value:
            for req in list(self._live):  # requests never waited for: finish and release them first
                self.wait(_V(req))
            check(lib.hc_h2h_destroy(self.handle), "hc_h2h_destroy")
            self.handle = _V()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cache_fingerprint(desc, model: str, tp_size: int) -> int:
    out = ctypes.c_uint64()
    check(lib.hc_cache_fingerprint(ctypes.byref(desc), model.encode(), tp_size, ctypes.byref(out)),
          "hc_cache_fingerprint")
    return out.value
