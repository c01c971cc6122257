"""Test rig for the GPU path: torch device pools, a pinned host pool, a copy stream
and an hc pool, plus comparisons against the oracle.  Test infrastructure."""
from __future__ import annotations

import sys

import numpy as np
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from oracle import oracle as O


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def geom_of(shape: W.PoolShape) -> O.Geometry:
    return O.Geometry(shape.layers, shape.page_size, [tuple(s) for s in shape.subs], shape.host_pages,
                      shape.device_slots, shape.layout, shape.align)


# Budget for page-locked host memory in one test process; a pool that does not fit
# keeps its rows, burst and device side and gets fewer host pages.
PIN_BUDGET = 64 << 30


def fit_pinned(shape: W.PoolShape, budget: int = PIN_BUDGET) -> W.PoolShape:
    """The same pool with as many host pages as fit the pinned-memory budget."""
    one = O.host_pool_bytes(O.Geometry(shape.layers, shape.page_size, [tuple(s) for s in shape.subs], 1,
                                       shape.device_slots, shape.layout, shape.align))
    pages = min(shape.host_pages, budget // one)
    if pages == shape.host_pages:
        return shape
    return W.shape_scaled(shape, shape.name, host_pages=pages)


def units(shape: W.PoolShape, b: int) -> int:
    gran, _ = shape.subs[b]
    return shape.device_slots // shape.page_size if gran == W.PAGE_BLOCKS else shape.device_slots


class Rig:
    """Device pool [sub][layer] (torch uint8), pinned host pool, copy stream, hc pool."""

    def __init__(self, shape: W.PoolShape, *, seed: int = 0, write_back_mode: int = B.HC_MODE_ZEROCOPY,
                 staging_pages: int = 0, flags: int = 0, max_ctas: int = 0, host_fill: int | None = 0xA5,
                 fill_device: bool = True):
        torch.cuda.synchronize()
        self.shape = shape
        self.geom = geom_of(shape)
        L = shape.layers
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        self.dev = []
        for b, (_, e) in enumerate(shape.subs):
            t = torch.empty((L, units(shape, b) * e), dtype=torch.uint8, device="cuda")
            if fill_device:
                t.random_(0, 256, generator=gen)
            self.dev.append(t)
        probe, _keep = B.make_desc(layers=L, page_size=shape.page_size,
                                   subs=[(g, e, [1] * L) for g, e in shape.subs],
                                   device_slots=shape.device_slots, host_pages=shape.host_pages,
                                   layout=shape.layout, shard_align=shape.align)
        self.host_bytes = B.host_pool_bytes(probe)
        self.host = B.HostBuffer(self.host_bytes)
        if host_fill is not None:
            self.host.fill(host_fill)
        self.staging = None
        if staging_pages:
            img = B.staging_page_bytes(probe)
            self.staging = torch.empty(staging_pages * img, dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        self.pool = B.Pool(layers=L, page_size=shape.page_size, subs=list(shape.subs),
                           device_slots=shape.device_slots, host_pages=shape.host_pages,
                           device_layers=[[self.dev[b][l] for l in range(L)] for b in range(len(shape.subs))],
                           host=self.host, stream=self.stream, layout=shape.layout, shard_align=shape.align,
                           staging=self.staging, write_back_mode=write_back_mode, flags=flags, max_ctas=max_ctas)

    def dev_np(self):
        return [[self.dev[b][l].cpu().numpy() for l in range(self.shape.layers)] for b in range(len(self.shape.subs))]

    def close(self):
        self.pool.close()
        self.host.free()
        self.dev = None
        self.staging = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def cuda_i64(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).cuda()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    if np.array_equal(got, want):
        return
    diff = np.flatnonzero(got != want)
    raise AssertionError(f"{what}: {diff.size} bytes differ, first at byte {diff[0]} "
                         f"(got {got[diff[0]]}, want {want[diff[0]]})")


def assert_dev_equal(got, want, what: str):
    for b in range(len(want)):
        for l in range(len(want[b])):
            assert_bytes_equal(got[b][l], want[b][l], f"{what}: sub {b} layer {l}")


def write_back_and_check(rig: Rig, d: np.ndarray, h: np.ndarray):
    """Write-back through the library; the whole host pool must equal the oracle's."""
    dev0 = rig.dev_np()
    host0 = rig.host.np.copy()
    d_t = cuda_i64(d)
    torch.cuda.synchronize()
    rig.pool.write_back_all_layers(d_t, np.ascontiguousarray(h, dtype=np.int64))
    rig.pool.sync()
    want = host0.copy()
    O.write_back(rig.geom, dev0, want, d, h)
    assert_bytes_equal(rig.host.np, want, "host pool after write-back")
    assert_dev_equal(rig.dev_np(), dev0, "device pool changed by write-back")


def load_back_and_check(rig: Rig, h: np.ndarray, d: np.ndarray, layers=None):
    """Per-layer load-back through the library; the whole device pool must equal the oracle's."""
    L = rig.shape.layers
    layers = list(range(L)) if layers is None else layers
    dev0 = rig.dev_np()
    host0 = rig.host.np.copy()
    h_t, d_t = cuda_i64(h), cuda_i64(d)
    torch.cuda.synchronize()
    events = [B.HipEvent() for _ in layers]
    for ev, l in zip(events, layers):
        rig.pool.load_back_layer(l, h_t, d_t, ev)
    for ev in events:
        ev.synchronize()
    rig.pool.sync()
    want = [[a.copy() for a in row] for row in dev0]
    for l in layers:
        O.load_back_layer(rig.geom, l, want, host0, h, d)
    assert_dev_equal(rig.dev_np(), want, "device pool after load-back")
    assert_bytes_equal(rig.host.np, host0, "host pool changed by load-back")
