"""GPU path at the workloads' full sizes, in the launch configuration the benchmark times.

Write-back: every named row (and page block) is compared bit-exactly with the device row
it came from (the oracle gives each row's host offset); every other byte of the whole
pinned host pool must still hold the fill, and the pads of touched shards must be zero
(the pool is streamed to the device in 1 GiB chunks and compared there under a mask of
the named rows); the device pool must equal a device-side copy taken before the call.
Load-back: every named slot of every layer equals its host row; every other slot of
every layer equals the device-side copy taken before the burst; the host pool outside
the named rows still holds the fill.
The 78-layer MLA + DSA indexer workload runs its per-layer load-back with a consumer on a
second stream that waits on each layer-done event and copies that layer's loaded rows;
each copy must equal the host rows element by element."""
import ctypes

import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, fit_pinned, say
from oracle import oracle as O

FILL = 0xA5
CHUNK = 1 << 30


def _hip():
    hip = B._hip
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    return hip


def host_rows(rig, b, layer, h):
    """Host bytes of the rows (or page blocks) named by h, as an (m, E) uint8 array."""
    gran, e = rig.shape.subs[b]
    if gran == W.PAGE_BLOCKS:
        h = h[h % rig.shape.page_size == 0]
    offs = O.host_offsets(rig.geom, b, layer, h)
    v16 = rig.host.np.view("V16")
    idx = (offs // 16)[:, None] + np.arange(e // 16)[None, :]
    return v16[idx].view(np.uint8).reshape(-1, e)


def dev_rows(rig, b, layer, d, h):
    gran, e = rig.shape.subs[b]
    if gran == W.PAGE_BLOCKS:
        d = d[h % rig.shape.page_size == 0] // rig.shape.page_size
    return rig.dev[b][layer].view(-1, e)[cuda_i64(d)].cpu().numpy()


def check_all_rows(rig, d, h, what):
    for b in range(len(rig.shape.subs)):
        for l in range(rig.shape.layers):
            got, want = host_rows(rig, b, l, h), dev_rows(rig, b, l, d, h)
            if not np.array_equal(got, want):
                bad = np.flatnonzero((got != want).any(axis=1))
                raise AssertionError(f"{what}: sub {b} layer {l}: {bad.size} rows differ, first token {bad[0]}")


def check_host_outside_named(rig, h, what):
    """Every byte of the whole host pool outside the rows and page blocks that h names holds
    the fill; the pads of the shards h touches are zero, the other pads hold the fill."""
    shape, g = rig.shape, rig.geom
    P, H = shape.page_size, shape.host_pages
    hip = _hip()
    named = torch.zeros(H * P, dtype=torch.bool, device="cuda")
    named[cuda_i64(h)] = True
    named = named.view(H, P)
    touched = named.any(1)
    buf = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    base = rig.host.ptr.value

    def load(off, n):
        torch.cuda.synchronize()
        assert hip.hipMemcpy(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(base + off), n, 1) == 0
        return buf[:n]

    def check_sub(x, b, p0, p1):
        gran, e = shape.subs[b]
        k = p1 - p0
        bad = x != FILL                                         # [k, sub page bytes], contiguous
        if gran == W.PAGE_BLOCKS:
            rows = bad.view(k, -1).any(1)
            ok = not bool((rows & ~named[p0:p1, 0]).any())
        elif shape.layout == W.PAGE_FIRST_TOKEN_MAJOR:
            rows = bad.view(k, P, -1).any(2)                    # [page][row][layer * elem]
            ok = not bool((rows & ~named[p0:p1]).any())
        else:
            rows = bad.view(k, shape.layers, P, e).any(3).any(1)  # [page][layer][row][elem]
            ok = not bool((rows & ~named[p0:p1]).any())
        assert ok, f"{what}: bytes outside the named rows changed (sub {b}, pages {p0}..{p1 - 1})"

    if shape.layout == W.KV_SPLIT_SHARD:
        stride, payload = O.shard_bytes(g), O.page_payload_bytes(g)
        per = max(1, CHUNK // stride)
        for p0 in range(0, H, per):
            p1 = min(H, p0 + per)
            x = load(p0 * stride, (p1 - p0) * stride).view(p1 - p0, stride)
            for b in range(len(shape.subs)):
                st, n = O.host_offset(g, b, 0, 0, 0), O.sub_page_bytes(g, b)
                check_sub(x[:, st:st + n], b, p0, p1)
            if stride > payload:
                pad = x[:, payload:]
                t = touched[p0:p1]
                assert not bool(pad[t].any()), f"{what}: a touched shard's pad is not zero"
                assert bool((pad[~t] == FILL).all()), f"{what}: an untouched shard's pad changed"
    else:
        for b in range(len(shape.subs)):
            region, sp = O.host_offset(g, b, 0, 0, 0), O.sub_page_bytes(g, b)
            per = max(1, CHUNK // sp)
            for p0 in range(0, H, per):
                p1 = min(H, p0 + per)
                check_sub(load(region + p0 * sp, (p1 - p0) * sp).view(p1 - p0, sp), b, p0, p1)
    del buf
    return int((~named[touched]).sum())  # rows of touched pages the list does not name


def device_copy(rig):
    return [t.clone() for t in rig.dev]


def check_device_unchanged(rig, before, what):
    for b in range(len(before)):
        assert torch.equal(rig.dev[b], before[b]), f"{what}: the device pool changed (sub {b})"


def check_device_outside(rig, before, d, h, what):
    """Every slot (or block) of every layer that d does not name equals its copy in `before`."""
    P = rig.shape.page_size
    for b, (gran, e) in enumerate(rig.shape.subs):
        units = rig.dev[b].shape[1] // e
        idx = d[h % P == 0] // P if gran == W.PAGE_BLOCKS else d
        keep = torch.ones(units, dtype=torch.bool, device="cuda")
        keep[cuda_i64(idx)] = False
        for l in range(rig.shape.layers):
            diff = (rig.dev[b][l] != before[b][l]).view(units, e).any(1)
            assert not bool((diff & keep).any()), f"{what}: unnamed device rows changed (sub {b} layer {l})"


def round_trip(rig, burst, d2):
    """Per-layer load-back of the burst's host rows into fresh slots, then checks."""
    h, d = burst.host_idx, burst.device_idx
    before = device_copy(rig)
    h_t, d2_t = cuda_i64(h), cuda_i64(d2)
    events = [B.HipEvent() for _ in range(rig.shape.layers)]
    torch.cuda.synchronize()
    for l in range(rig.shape.layers):
        rig.pool.load_back_layer(l, h_t, d2_t, events[l])
    rig.pool.sync()
    for b in range(len(rig.shape.subs)):
        for l in range(rig.shape.layers):
            got, want = dev_rows(rig, b, l, d2, h), host_rows(rig, b, l, h)
            assert np.array_equal(got, want), f"load-back sub {b} layer {l} differs"
    check_device_outside(rig, before, d2, h, "load-back")
    del before
    check_host_outside_named(rig, h, "host pool after the load-back")
    assert rig.pool.round_trip_check(cuda_i64(d), d2_t) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("name,mode", [
    ("llama3_8b_mha_bf16", "zerocopy"),
    ("llama3_8b_mha_bf16", "staged"),
    ("llama3_8b_mha_bf16_token_major", "zerocopy"),
    ("llama3_8b_mha_bf16_token_major", "staged"),
    ("dsv3_mla_bf16", "zerocopy"),
    ("dsv3_mla_bf16", "staged"),
    ("dsa_mla_indexer_78l", "zerocopy"),
    ("dsa_mla_indexer_78l", "staged"),
    ("mha_kv_split_shard_bf16", "zerocopy"),
    ("mha_kv_split_shard_bf16", "staged"),
])
def test_full_size_write_back_and_load_back(name, mode):
    shape = fit_pinned(W.SHAPES[name])
    say(f"[full] {name} mode={mode}: building pools (host pages {shape.host_pages} of {W.SHAPES[name].host_pages})")
    wb = B.HC_MODE_STAGED if mode == "staged" else B.HC_MODE_ZEROCOPY
    rig = Rig(shape, seed=3, write_back_mode=wb, staging_pages=64 if mode == "staged" else 0, host_fill=FILL)
    try:
        burst = W.burst_for(shape, seed=1)
        say(f"[full] {name}: write-back of {burst.n} tokens, {burst.pages.size} pages")
        before = device_copy(rig)
        torch.cuda.synchronize()
        rig.pool.write_back_all_layers(cuda_i64(burst.device_idx), burst.host_idx)
        rig.pool.sync()
        check_device_unchanged(rig, before, f"{name} write-back")
        del before
        check_all_rows(rig, burst.device_idx, burst.host_idx, f"{name} write-back")
        unnamed = check_host_outside_named(rig, burst.host_idx, f"{name} write-back")
        if name == "mha_kv_split_shard_bf16":
            assert unnamed > 0, "the shard workload must name partial pages"
        say(f"[full] {name}: load-back")
        round_trip(rig, burst, W.fresh_slots_like(shape, burst, seed=2))
    finally:
        rig.close()


def fill_host_random(rig, seed):
    """Seeded random bytes into the whole host pool: torch draws them on the device,
    hipMemcpy carries them over (plumbing, not the transfer path)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    buf = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    hip = _hip()
    for off in range(0, rig.host.nbytes, CHUNK):
        n = min(CHUNK, rig.host.nbytes - off)
        buf.random_(0, 256, generator=gen)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(ctypes.c_void_p(rig.host.ptr.value + off), ctypes.c_void_p(buf.data_ptr()), n, 2) == 0
    del buf


@pytest.mark.gpu
def test_full_size_mla_indexer_load_back_with_consumer():
    """78 layers, latent rows + indexer page blocks in one burst of 1024 pages; a consumer
    stream waits on each layer-done event, then copies that layer's loaded rows and blocks.
    Every copy must equal the host rows element by element, and every slot the burst does
    not name must keep its bytes."""
    shape = fit_pinned(W.SHAPES["dsa_mla_indexer_78l"])
    say("[full] dsa_mla_indexer_78l: building pools")
    rig = Rig(shape, seed=4, host_fill=None)
    try:
        fill_host_random(rig, seed=44)
        burst = W.burst_for(shape, seed=1, purpose="load_back")
        h, d = burst.host_idx, burst.device_idx
        P = shape.page_size
        before = device_copy(rig)
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        blk_t = cuda_i64(d[h % P == 0] // P)
        consumer = torch.cuda.Stream()
        events = [B.HipEvent() for _ in range(shape.layers)]
        seen = []
        torch.cuda.synchronize()
        say(f"[full] dsa_mla_indexer_78l: load-back of {burst.n} tokens x {shape.layers} layers")
        for l in range(shape.layers):
            rig.pool.load_back_layer(l, h_t, d_t, events[l])
            events[l].wait_on(consumer)
            with torch.cuda.stream(consumer):
                lat = rig.dev[0][l].view(-1, shape.subs[0][1])[d_t].clone()
                idx = rig.dev[1][l].view(-1, shape.subs[1][1])[blk_t].clone()
                seen.append((lat, idx))
        consumer.synchronize()
        rig.pool.sync()
        for l in range(shape.layers):
            assert np.array_equal(seen[l][0].cpu().numpy(), host_rows(rig, 0, l, h)), \
                f"consumer saw other latent rows in layer {l}"
            assert np.array_equal(seen[l][1].cpu().numpy(), host_rows(rig, 1, l, h)), \
                f"consumer saw other indexer blocks in layer {l}"
        for b in range(2):
            for l in range(shape.layers):
                assert np.array_equal(dev_rows(rig, b, l, d, h), host_rows(rig, b, l, h)), (b, l)
        check_device_outside(rig, before, d, h, "78-layer load-back")
    finally:
        rig.close()
