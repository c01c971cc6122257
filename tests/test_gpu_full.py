"""GPU path at the workloads' full sizes, in the launch configuration the benchmark times.

Every row of the burst is compared bit-exactly: the oracle gives each row's host
offset, torch gathers the expected device rows, numpy gathers the host rows.
Untouched host pages and device slots are sampled.  The 78-layer MLA + DSA
indexer workload runs its per-layer load-back with a consumer on a second
stream that waits on each layer-done event and checksums the layer."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, fit_pinned, say
from oracle import oracle as O

FILL = 0xA5


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


def check_untouched_pages(rig, h, samples=24, seed=0):
    P = rig.shape.page_size
    named = np.unique(h // P)
    free = np.setdiff1d(np.arange(rig.shape.host_pages), named)
    pick = np.random.default_rng(seed).choice(free, size=min(samples, free.size), replace=False)
    for p in pick:
        for b in range(len(rig.shape.subs)):
            st = O.host_offset(rig.geom, b, int(p), 0, 0)
            n = O.sub_page_bytes(rig.geom, b)
            assert (rig.host.np[st:st + n] == FILL).all(), f"untouched page {p} sub {b} changed"


def check_partial_pages(rig, h):
    """Rows of touched pages that the list does not name keep the fill; pads are zero."""
    P = rig.shape.page_size
    pages = np.unique(h // P)
    every = (pages[:, None] * P + np.arange(P)[None, :]).reshape(-1)
    unnamed = np.setdiff1d(every, h)
    for b, (gran, e) in enumerate(rig.shape.subs):
        if gran == W.PAGE_BLOCKS or unnamed.size == 0:
            continue
        for l in range(rig.shape.layers):
            rows = host_rows(rig, b, l, unnamed)
            assert (rows == FILL).all(), f"unnamed rows of touched pages changed (sub {b} layer {l})"
    if rig.shape.layout == W.KV_SPLIT_SHARD:
        stride = O.shard_bytes(rig.geom)
        payload = O.page_payload_bytes(rig.geom)
        for p in pages:
            assert not rig.host.np[p * stride + payload:(p + 1) * stride].any(), f"pad of shard {p} not zero"
    return unnamed.size


def sample_slots(rig, exclude, k=4096, seed=1):
    free = np.setdiff1d(np.arange(rig.shape.device_slots), exclude)
    return np.random.default_rng(seed).choice(free, size=min(k, free.size), replace=False)


def snapshot(rig, slots):
    out = []
    for b, (gran, e) in enumerate(rig.shape.subs):
        s = slots // rig.shape.page_size if gran == W.PAGE_BLOCKS else slots
        s = np.unique(s)
        out.append([rig.dev[b][l].view(-1, e)[cuda_i64(s)].cpu().numpy() for l in range(rig.shape.layers)])
    return out


def round_trip(rig, burst, d2):
    """Per-layer load-back of the burst's host rows into fresh slots, then checks."""
    h, d = burst.host_idx, burst.device_idx
    keep = sample_slots(rig, np.concatenate([d2, d]))
    before = snapshot(rig, keep)
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
    after = snapshot(rig, keep)
    for b in range(len(before)):
        for l in range(len(before[b])):
            assert np.array_equal(before[b][l], after[b][l]), f"untouched device slots changed (sub {b} layer {l})"
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
        torch.cuda.synchronize()
        rig.pool.write_back_all_layers(cuda_i64(burst.device_idx), burst.host_idx)
        rig.pool.sync()
        check_all_rows(rig, burst.device_idx, burst.host_idx, f"{name} write-back")
        check_untouched_pages(rig, burst.host_idx)
        unnamed = check_partial_pages(rig, burst.host_idx)
        if name == "mha_kv_split_shard_bf16":
            assert unnamed > 0, "the shard workload must name partial pages"
        say(f"[full] {name}: load-back")
        round_trip(rig, burst, W.fresh_slots_like(shape, burst, seed=2))
    finally:
        rig.close()


def fill_host_random(rig, seed):
    """Seeded random bytes into the whole host pool: torch draws them on the device,
    hipMemcpy carries them over (plumbing, not the transfer path)."""
    import ctypes
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    chunk = 1 << 30
    buf = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    hip = B._hip
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    for off in range(0, rig.host.nbytes, chunk):
        n = min(chunk, rig.host.nbytes - off)
        buf.random_(0, 256, generator=gen)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(ctypes.c_void_p(rig.host.ptr.value + off), ctypes.c_void_p(buf.data_ptr()), n, 2) == 0
    del buf


def checksum_np(rows):
    return int(rows.view(np.int32).astype(np.int64).sum())


@pytest.mark.gpu
def test_full_size_mla_indexer_load_back_with_consumer():
    """78 layers, latent rows + indexer page blocks in one burst of 1024 pages; a consumer
    stream waits on each layer-done event, then checksums that layer's loaded rows."""
    shape = fit_pinned(W.SHAPES["dsa_mla_indexer_78l"])
    say("[full] dsa_mla_indexer_78l: building pools")
    rig = Rig(shape, seed=4, host_fill=None)
    try:
        fill_host_random(rig, seed=44)
        burst = W.burst_for(shape, seed=1, purpose="load_back")
        h, d = burst.host_idx, burst.device_idx
        P = shape.page_size
        keep = sample_slots(rig, d)
        before = snapshot(rig, keep)
        h_t, d_t = cuda_i64(h), cuda_i64(d)
        blk_t = cuda_i64(d[h % P == 0] // P)
        consumer = torch.cuda.Stream()
        events = [B.HipEvent() for _ in range(shape.layers)]
        sums = []
        torch.cuda.synchronize()
        say(f"[full] dsa_mla_indexer_78l: load-back of {burst.n} tokens x {shape.layers} layers")
        for l in range(shape.layers):
            rig.pool.load_back_layer(l, h_t, d_t, events[l])
            events[l].wait_on(consumer)
            with torch.cuda.stream(consumer):
                lat = rig.dev[0][l].view(-1, shape.subs[0][1])[d_t].view(torch.int32).to(torch.int64).sum()
                idx = rig.dev[1][l].view(-1, shape.subs[1][1])[blk_t].view(torch.int32).to(torch.int64).sum()
                sums.append((lat, idx))
        consumer.synchronize()
        rig.pool.sync()
        for l in range(shape.layers):
            want_lat = checksum_np(host_rows(rig, 0, l, h))
            want_idx = checksum_np(host_rows(rig, 1, l, h))
            assert int(sums[l][0]) == want_lat, f"consumer saw stale latent rows in layer {l}"
            assert int(sums[l][1]) == want_idx, f"consumer saw stale indexer blocks in layer {l}"
        for b in range(2):
            for l in range(shape.layers):
                assert np.array_equal(dev_rows(rig, b, l, d, h), host_rows(rig, b, l, h)), (b, l)
        after = snapshot(rig, keep)
        for b in range(2):
            for l in range(shape.layers):
                assert np.array_equal(before[b][l], after[b][l]), f"untouched slots changed ({b}, {l})"
    finally:
        rig.close()
