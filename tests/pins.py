"""Pins for the oracle: checks against formulations that do not share its arithmetic.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
  * a structural brute force (the host pool is rebuilt by walking pages,
    sub-buffers, layers and rows in layout order and concatenating byte
    strings; positions come from running sums, never from an offset formula),
  * the CPU mock formula of the hybrid-pool write-back page (key source
    excerpts: for every layer, host[dst_index, layer] = device_layer[src_index])
    written with numpy fancy indexing on a 4-d view,
  * invariants: a write-back followed by a load-back into fresh slots restores
    every row bit-exactly, untouched rows and pages keep their bytes, shard pad
    bytes become zero (CacheStore H2H page, "page_first_kv_split support"),
  * closed forms worked out by hand in ``golden/layout_closed_forms.txt``,
  * for the per-layer exchange of a rank-sharded tier (rank-sharded tier page,
    Modifications and Accuracy Tests): numpy gathers of the loaded rows, and two
    replicas of a pool that agree again after every layer's exchange.

``run_all()`` runs every pin; the mutation test runs it in a subprocess
against deliberately broken builds of the oracle and expects a failure.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402

T, B = O.TOKEN_ROWS, O.PAGE_BLOCKS
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "layout_closed_forms.txt")

# Tiny geometries: both layouts, token rows and page blocks, nonzero shard pad.
GEOMS = {
    "pf_kv": O.Geometry(2, 4, [(T, 32), (T, 32)], 6, 64, O.PAGE_FIRST),
    "pf_one": O.Geometry(3, 4, [(T, 48)], 5, 40, O.PAGE_FIRST),
    "shard_kv_pad": O.Geometry(3, 4, [(T, 32), (T, 16)], 6, 64, O.KV_SPLIT_SHARD, align=256),
    "pf_latent_indexer": O.Geometry(2, 4, [(T, 32), (B, 48)], 6, 64, O.PAGE_FIRST),
    "shard_block_pad": O.Geometry(2, 4, [(T, 16), (B, 32)], 5, 32, O.KV_SPLIT_SHARD, align=128),
    "tm_kv": O.Geometry(3, 4, [(T, 32), (T, 16)], 6, 64, O.PAGE_FIRST_TOKEN_MAJOR),
    "tm_latent_indexer": O.Geometry(2, 4, [(T, 32), (B, 48)], 6, 64, O.PAGE_FIRST_TOKEN_MAJOR),
}


def has_blocks(g: O.Geometry) -> bool:
    return any(gr == B for gr, _ in g.subs)


# ---------------------------------------------------------------- structural model
def layout_walk(g: O.Geometry):
    """Yield (key, nbytes) for every piece of the host pool in storage order.
    key = ("row", b, p, l, r) for a token row, ("blk", b, p, l) for a page block,
    ("pad", p) for shard padding."""

    def page_pieces(b, p):
        gran, e = g.subs[b]
        if gran == B:
            for l in range(g.layers):
                yield ("blk", b, p, l), e
        elif g.layout == O.PAGE_FIRST_TOKEN_MAJOR:
            for r in range(g.page_size):
                for l in range(g.layers):
                    yield ("row", b, p, l, r), e
        else:
            for l in range(g.layers):
                for r in range(g.page_size):
                    yield ("row", b, p, l, r), e

    if g.layout in (O.PAGE_FIRST, O.PAGE_FIRST_TOKEN_MAJOR):
        for b in range(len(g.subs)):
            for p in range(g.host_pages):
                yield from page_pieces(b, p)
    else:
        payload = 0
        for b in range(len(g.subs)):
            for _, e in page_pieces(b, 0):
                payload += e
        pad = (-payload) % g.align
        for p in range(g.host_pages):
            for b in range(len(g.subs)):
                yield from page_pieces(b, p)
            yield ("pad", p), pad


def positions(g: O.Geometry) -> dict:
    """key -> (start, nbytes), by running sum over the storage order."""
    pos, at = {}, 0
    for key, n in layout_walk(g):
        pos[key] = (at, n)
        at += n
    return pos, at


def random_device(g: O.Geometry, rng) -> list:
    return [[rng.integers(0, 256, g.device_units(b) * e, dtype=np.uint8) for _ in range(g.layers)]
            for b, (_, e) in enumerate(g.subs)]


def copy_device(dev) -> list:
    return [[a.copy() for a in layers] for layers in dev]


def make_burst(g: O.Geometry, rng, partial: bool = True):
    """Distinct host pages; whole pages, plus (token-row pools only) one partial page
    missing some rows; device slots distinct (page-aligned whole pages for block pools)."""
    P = g.page_size
    npages = max(1, g.host_pages // 2)
    pages = rng.choice(g.host_pages, size=npages, replace=False)
    toks = []
    for j, p in enumerate(pages):
        rows = np.arange(P)
        if partial and not has_blocks(g) and j == len(pages) - 1 and P > 1:
            rows = np.sort(rng.choice(P, size=P - 1, replace=False))
        toks.append(p * P + rows)
    h = np.concatenate(toks).astype(np.int64)
    if has_blocks(g):
        dpages = rng.choice(g.device_slots // P, size=npages, replace=False)
        d = (dpages[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
    else:
        d = rng.choice(g.device_slots, size=h.size, replace=False).astype(np.int64)
    return d, h


def fresh_slots(g: O.Geometry, rng, used: np.ndarray, n: int) -> np.ndarray:
    P = g.page_size
    if has_blocks(g):
        free = np.setdiff1d(np.arange(g.device_slots // P), np.unique(used // P))
        dp = rng.choice(free, size=n // P, replace=False)
        return (dp[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
    free = np.setdiff1d(np.arange(g.device_slots), used)
    return rng.choice(free, size=n, replace=False).astype(np.int64)


def expected_host_after_write_back(g, dev, host0: np.ndarray, d, h) -> np.ndarray:
    """Brute force: walk the layout, and for every piece decide its bytes."""
    P = g.page_size
    named = {int(hh): int(dd) for dd, hh in zip(d, h)}
    touched = {int(hh) // P for hh in h}
    out, at = [], 0
    for key, n in layout_walk(g):
        cur = host0[at:at + n].tobytes()
        if key[0] == "row":
            _, b, p, l, r = key
            if p * P + r in named:
                s = named[p * P + r]
                e = g.subs[b][1]
                cur = dev[b][l][s * e:(s + 1) * e].tobytes()
        elif key[0] == "blk":
            _, b, p, l = key
            if p * P in named:
                blk = named[p * P] // P
                e = g.subs[b][1]
                cur = dev[b][l][blk * e:(blk + 1) * e].tobytes()
        else:
            _, p = key
            if p in touched:
                cur = bytes(n)
        out.append(cur)
        at += n
    return np.frombuffer(b"".join(out), dtype=np.uint8).copy()


def expected_device_after_load_back(g, layer, dev0, host: np.ndarray, h, d):
    pos, _ = positions(g)
    P = g.page_size
    dev = copy_device(dev0)
    for dd, hh in zip(d, h):
        p, r = int(hh) // P, int(hh) % P
        for b, (gran, e) in enumerate(g.subs):
            if gran == B:
                if r != 0:
                    continue
                st, n = pos[("blk", b, p, layer)]
                blk = int(dd) // P
                dev[b][layer][blk * e:(blk + 1) * e] = host[st:st + n]
            else:
                st, n = pos[("row", b, p, layer, r)]
                dev[b][layer][int(dd) * e:(int(dd) + 1) * e] = host[st:st + n]
    return dev


def assert_dev_equal(x, y, what=""):
    for b in range(len(x)):
        for l in range(len(x[b])):
            assert np.array_equal(x[b][l], y[b][l]), f"{what}: sub {b} layer {l} differs"


# ---------------------------------------------------------------- pins
def pin_sizes_match_structure():
    for name, g in GEOMS.items():
        _, total = positions(g)
        assert O.host_pool_bytes(g) == total, name
        if g.layout == O.KV_SPLIT_SHARD:
            assert total % g.host_pages == 0
            stride = total // g.host_pages
            assert O.shard_bytes(g) == stride, name
            assert stride % g.align == 0, name
            assert stride - O.page_payload_bytes(g) < g.align, name


def pin_offsets_match_structure():
    for name, g in GEOMS.items():
        pos, _ = positions(g)
        for key, (st, _) in pos.items():
            if key[0] == "row":
                _, b, p, l, r = key
                assert O.host_offset(g, b, p, l, r) == st, (name, key)
            elif key[0] == "blk":
                _, b, p, l = key
                for r in (0, g.page_size - 1):
                    assert O.host_offset(g, b, p, l, r) == st, (name, key, r)


def pin_write_back_brute_force():
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(100 + seed)
        dev = random_device(g, rng)
        host0 = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng)
        want = expected_host_after_write_back(g, dev, host0, d, h)
        host = host0.copy()
        dev_before = copy_device(dev)
        O.write_back(g, dev, host, d, h)
        assert np.array_equal(host, want), name
        assert_dev_equal(dev, dev_before, f"{name}: write-back changed the device pool")


def pin_write_back_mock_formula():
    """host4[page, layer, row] = device_layer[slot], per layer, on 4-d views."""
    for seed, (name, g) in enumerate(GEOMS.items()):
        if has_blocks(g):
            continue
        rng = np.random.default_rng(200 + seed)
        dev = random_device(g, rng)
        host = np.zeros(O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng)
        O.write_back(g, dev, host, d, h)
        want = np.zeros_like(host)
        L, P, H = g.layers, g.page_size, g.host_pages
        page, row = h // P, h % P
        if g.layout == O.PAGE_FIRST_TOKEN_MAJOR:
            # the mock's own indexing: host[token, layer] = device_layer[slot]
            start = 0
            for b, (_, e) in enumerate(g.subs):
                region = want[start:start + H * P * L * e].reshape(H * P, L, e)
                for l in range(L):
                    region[h, l] = dev[b][l].reshape(-1, e)[d]
                start += H * P * L * e
        elif g.layout == O.PAGE_FIRST:
            start = 0
            for b, (_, e) in enumerate(g.subs):
                region = want[start:start + H * L * P * e].reshape(H, L, P, e)
                for l in range(L):
                    region[page, l, row] = dev[b][l].reshape(-1, e)[d]
                start += H * L * P * e
        else:
            payload = sum(L * P * e for _, e in g.subs)
            stride = payload + (-payload) % g.align
            shards = want.reshape(H, stride)
            start = 0
            for b, (_, e) in enumerate(g.subs):
                view = shards[:, start:start + L * P * e].reshape(H, L, P, e)
                for l in range(L):
                    view[page, l, row] = dev[b][l].reshape(-1, e)[d]
                start += L * P * e
        assert np.array_equal(host, want), name


def pin_load_back_brute_force():
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(300 + seed)
        dev0 = random_device(g, rng)
        host = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        host_before = host.copy()
        d, h = make_burst(g, rng)
        for layer in range(g.layers):
            want = expected_device_after_load_back(g, layer, dev0, host, h, d)
            dev = copy_device(dev0)
            O.load_back_layer(g, layer, dev, host, h, d)
            assert_dev_equal(dev, want, f"{name} layer {layer}")
        assert np.array_equal(host, host_before), f"{name}: load-back changed the host pool"


def pin_round_trip_restores():
    """Write back all layers, then load every layer into fresh slots: rows equal."""
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(400 + seed)
        dev = random_device(g, rng)
        host = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng)
        O.write_back(g, dev, host, d, h)
        dev_before = copy_device(dev)
        d2 = fresh_slots(g, rng, d, d.size)
        for layer in range(g.layers):
            O.load_back_layer(g, layer, dev, host, h, d2)
        P = g.page_size
        for b, (gran, e) in enumerate(g.subs):
            for l in range(g.layers):
                a = dev[b][l].reshape(-1, e)
                a0 = dev_before[b][l].reshape(-1, e)
                src = d // P if gran == B else d
                dst = d2 // P if gran == B else d2
                assert np.array_equal(a[dst], a0[src]), (name, b, l)
                untouched = np.setdiff1d(np.arange(a.shape[0]), dst)
                assert np.array_equal(a[untouched], a0[untouched]), (name, b, l)
        assert O.round_trip_check(g, dev, d, d2) == 0, name


def pin_untouched_and_byte_accounting():
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(500 + seed)
        dev = random_device(g, rng)
        host0 = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng)
        host = host0.copy()
        O.write_back(g, dev, host, d, h)
        pos, _ = positions(g)
        P = g.page_size
        named = set(int(x) for x in h)
        touched = set(int(x) // P for x in h)
        changed_allowed = np.zeros(host.size, dtype=bool)
        for key, (st, n) in pos.items():
            if key[0] == "row" and key[2] * P + key[4] in named:
                changed_allowed[st:st + n] = True
            if key[0] == "blk" and key[2] * P in named:
                changed_allowed[st:st + n] = True
            if key[0] == "pad" and key[1] in touched:
                changed_allowed[st:st + n] = True
                assert not host[st:st + n].any(), (name, "pad not zero")
        assert np.array_equal(host[~changed_allowed], host0[~changed_allowed]), name
        row_bytes = sum(e * g.layers for gran, e in g.subs if gran == T) * len(named)
        blk_bytes = sum(e * g.layers for gran, e in g.subs if gran == B) * len(touched)
        pad_bytes = sum(n for k, (st, n) in pos.items() if k[0] == "pad" and k[1] in touched)
        assert int((host != host0).sum()) <= row_bytes + blk_bytes + pad_bytes, name


def pin_round_trip_check_counts():
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(600 + seed)
        dev = random_device(g, rng)
        d, _ = make_burst(g, rng, partial=False)
        c = fresh_slots(g, rng, d, d.size)
        # make a known set of units equal: copy rows of d onto c for some units
        P = g.page_size
        want = 0
        for b, (gran, e) in enumerate(g.subs):
            for l in range(g.layers):
                a = dev[b][l].reshape(-1, e)
                for i in range(d.size):
                    if gran == B and d[i] % P != 0:
                        continue
                    x = d[i] // P if gran == B else d[i]
                    y = c[i] // P if gran == B else c[i]
                    if (i + l + b) % 3 == 0:
                        a[y] = a[x]
                    elif (i + l) % 5 == 0:
                        a[y] = a[x]
                        a[y, (i * 7 + l) % e] ^= 0x40
                        want += 1
                    else:
                        want += int(not np.array_equal(a[x], a[y]))
        assert O.round_trip_check(g, dev, d, c) == want, name


def pin_index_preconditions():
    g = GEOMS["pf_kv"]
    assert O.check_indices(g, [0, 1, 2], [0, 1, 2])
    assert not O.check_indices(g, [0, 0], [0, 1]), "repeated device slot accepted"
    assert not O.check_indices(g, [0, 1], [5, 5]), "repeated host token accepted"
    assert not O.check_indices(g, [g.device_slots], [0]), "device slot out of range accepted"
    assert not O.check_indices(g, [0], [g.host_pages * g.page_size]), "host token out of range accepted"
    assert not O.check_indices(g, [-1], [0]), "negative slot accepted"
    assert O.check_indices(g, [], [])
    gb = GEOMS["pf_latent_indexer"]
    P = gb.page_size
    whole = np.arange(P)
    assert O.check_indices(gb, 8 + whole, 2 * P + whole)
    assert not O.check_indices(gb, 8 + whole[:-1], 2 * P + whole[:-1]), "partial block page accepted"
    assert not O.check_indices(gb, 9 + whole, 2 * P + whole), "misaligned device page accepted"
    assert not O.check_indices(gb, 8 + whole[::-1], 2 * P + whole), "reordered rows accepted"


def pin_golden_closed_forms():
    with open(GOLDEN) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) >= 20
    for ln in lines:
        name, geo, q = [x.strip() for x in ln.split("|")]
        layout, L, P, H, S, align, subs = geo.split()
        sub = [((T if s[0] == "T" else B), int(s[1:])) for s in subs.split(",")]
        lay = {"shard": O.KV_SPLIT_SHARD, "page_first": O.PAGE_FIRST, "token_major": O.PAGE_FIRST_TOKEN_MAJOR}[layout]
        g = O.Geometry(int(L), int(P), sub, int(H), int(S), lay, int(align))
        lhs, rhs = [x.strip() for x in q.split("=")]
        what, *args = lhs.split()
        args = [int(a) for a in args]
        fn = {"sub_page_bytes": O.sub_page_bytes, "payload_bytes": O.page_payload_bytes,
              "shard_bytes": O.shard_bytes, "host_pool_bytes": O.host_pool_bytes,
              "host_offset": O.host_offset, "device_offset": O.device_offset}[what]
        got = fn(g, *args)
        assert got == int(rhs), f"{name}: {lhs} = {got}, closed form {rhs}"


def pin_h2h_shard_dump_and_load():
    """Store shard = the host page's sub-buffer pages back to back (each taken in
    storage order from the page-first pool), then zeros to the shard size; a load
    puts the same bytes back; shards and pages not named keep their bytes."""
    cases = [([(T, 32), (T, 16)], 3, 4, 256), ([(T, 48), (B, 32)], 2, 4, 128), ([(T, 16)], 1, 1, 64)]
    for k, (subs, L, P, align) in enumerate(cases):
        rng = np.random.default_rng(700 + k)
        pf = O.Geometry(L, P, subs, 7, 64, O.PAGE_FIRST)
        sh = O.Geometry(L, P, subs, 5, 64, O.KV_SPLIT_SHARD, align=align)
        host = rng.integers(0, 256, O.host_pool_bytes(pf), dtype=np.uint8)
        store0 = rng.integers(0, 256, O.host_pool_bytes(sh), dtype=np.uint8)
        store = store0.copy()
        src, dst = np.array([6, 0, 3]), np.array([4, 1, 2])
        O.h2h_dump(pf, sh, host, store, src, dst)
        pos, _ = positions(pf)
        stride = O.host_pool_bytes(sh) // sh.host_pages
        for p, q in zip(src, dst):
            parts = []
            for b in range(len(subs)):
                keys = sorted((st, n) for key, (st, n) in pos.items() if key[0] in ("row", "blk")
                              and key[1] == b and key[2] == p)
                parts.append(b"".join(host[st:st + n].tobytes() for st, n in keys))
            img = b"".join(parts)
            want = img + bytes(stride - len(img))
            assert store[q * stride:(q + 1) * stride].tobytes() == want, (k, p, q)
        for q in set(range(sh.host_pages)) - set(dst.tolist()):
            assert np.array_equal(store[q * stride:(q + 1) * stride], store0[q * stride:(q + 1) * stride]), (k, q)
        back = rng.integers(0, 256, host.size, dtype=np.uint8)
        before = back.copy()
        O.h2h_load(pf, sh, back, store, dst, np.array([1, 5, 6]))
        page = O.sub_page_bytes
        for p_src, p_dst in zip(src, [1, 5, 6]):
            for b in range(len(subs)):
                a0 = O.host_offset(pf, b, int(p_src), 0, 0)
                a1 = O.host_offset(pf, b, int(p_dst), 0, 0)
                n = page(pf, b)
                assert np.array_equal(back[a1:a1 + n], host[a0:a0 + n]), (k, p_src, p_dst, b)
        for p_other in set(range(pf.host_pages)) - {1, 5, 6}:
            for b in range(len(subs)):
                a1 = O.host_offset(pf, b, p_other, 0, 0)
                n = page(pf, b)
                assert np.array_equal(back[a1:a1 + n], before[a1:a1 + n]), (k, p_other)


def pin_burst_algebra():
    """The copy has no hidden state: writing a burst back twice equals once; bursts on
    disjoint host pages commute; a burst equals its split into consecutive parts (the
    chunking a staged write-back does); load-back of disjoint device slots commutes."""
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(800 + seed)
        dev = random_device(g, rng)
        host0 = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng, partial=not has_blocks(g))
        once = host0.copy()
        O.write_back(g, dev, once, d, h)
        twice = once.copy()
        O.write_back(g, dev, twice, d, h)
        assert np.array_equal(once, twice), (name, "not idempotent")
        P = g.page_size
        pages = np.unique(h // P)
        half = set(pages[: max(1, pages.size // 2)].tolist())
        a = np.array([i for i in range(h.size) if h[i] // P in half])
        b = np.array([i for i in range(h.size) if h[i] // P not in half], dtype=np.int64)
        ab, ba = host0.copy(), host0.copy()
        O.write_back(g, dev, ab, d[a], h[a])
        O.write_back(g, dev, ab, d[b], h[b])
        O.write_back(g, dev, ba, d[b], h[b])
        O.write_back(g, dev, ba, d[a], h[a])
        assert np.array_equal(ab, ba), (name, "disjoint bursts do not commute")
        assert np.array_equal(ab, once), (name, "split burst differs from the whole burst")
        if not has_blocks(g):
            cut = h.size // 3
            parts = host0.copy()
            O.write_back(g, dev, parts, d[:cut], h[:cut])
            O.write_back(g, dev, parts, d[cut:], h[cut:])
            assert np.array_equal(parts, once), (name, "consecutive parts differ from the whole burst")
        d2 = fresh_slots(g, rng, d, d.size)
        x, y = copy_device(dev), copy_device(dev)
        for layer in range(g.layers):
            O.load_back_layer(g, layer, x, once, h[a], d2[a])
            O.load_back_layer(g, layer, x, once, h[b], d2[b])
        for layer in reversed(range(g.layers)):
            O.load_back_layer(g, layer, y, once, h[b], d2[b])
            O.load_back_layer(g, layer, y, once, h[a], d2[a])
        assert_dev_equal(x, y, f"{name}: load-back order")


# ---------------------------------------------------------------- layer exchange of a rank-sharded tier
def pin_layer_exchange_gather_formula():
    """Exchange staging (rank-sharded tier page, Modifications: the owner gathers a
    loaded layer's rows into a staging buffer) against numpy fancy indexing on
    [units, E] views of the device layer: sub-buffer after sub-buffer, token rows
    view[d], page blocks view[d[0::P] // P]; its size is the concatenation's."""
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(900 + seed)
        dev = random_device(g, rng)
        dev0 = copy_device(dev)
        d, _ = make_burst(g, rng)  # ragged n for token-row pools
        for layer in range(g.layers):
            parts = []
            for b, (gran, e) in enumerate(g.subs):
                view = dev[b][layer].reshape(-1, e)
                parts.append(view[d[0::g.page_size] // g.page_size] if gran == B else view[d])
            want = np.concatenate([x.reshape(-1) for x in parts])
            got = O.layer_pack(g, layer, dev, d)
            assert got.size == want.size == O.layer_packed_bytes(g, d.size), (name, layer)
            assert np.array_equal(got, want), f"{name} layer {layer}: staging differs from the gather"
        assert_dev_equal(dev, dev0, f"{name}: pack changed the device pool")
        assert O.layer_pack(g, 0, dev, np.zeros(0, np.int64)).size == 0


def pin_layer_exchange_restores_owner_rows():
    """Two replicas of one device pool (every TP rank holds the same slots).  Layer by
    layer the owner loads from its host pool, packs, and the other rank unpacks: the
    other rank's pool then equals the structural load-back of the same rows, bit for
    bit, with every other layer and slot untouched (the page's accuracy claim).  A
    skipped exchange, the page's negative control, leaves the replicas different."""
    for seed, (name, g) in enumerate(GEOMS.items()):
        rng = np.random.default_rng(950 + seed)
        owner = random_device(g, rng)
        other = copy_device(owner)
        host = rng.integers(0, 256, O.host_pool_bytes(g), dtype=np.uint8)
        d, h = make_burst(g, rng)
        want = copy_device(other)
        for layer in range(g.layers):
            want = expected_device_after_load_back(g, layer, want, host, h, d)
            O.load_back_layer(g, layer, owner, host, h, d)
            assert any(not np.array_equal(owner[b][layer], other[b][layer]) for b in range(len(g.subs))), \
                f"{name} layer {layer}: negative control not caught"
            O.layer_unpack(g, layer, other, d, O.layer_pack(g, layer, owner, d))
            assert_dev_equal(other, want, f"{name} after the exchange of layer {layer}")
        assert_dev_equal(other, owner, f"{name}: replicas differ after every exchange")


def pin_layer_exchange_preconditions():
    """Lists the exchange refuses: out-of-range or repeated slots, and with page blocks
    a count that is not whole pages, a page not starting at a multiple of P, rows of a
    page out of order.  Token-row pools take ragged and empty lists."""
    g = GEOMS["pf_latent_indexer"]
    P = g.page_size
    dev = random_device(g, np.random.default_rng(990))
    d = np.concatenate([p * P + np.arange(P) for p in (5, 0, 9)]).astype(np.int64)
    O.layer_pack(g, 1, dev, d)
    swapped = d.copy()
    swapped[[1, 2]] = swapped[[2, 1]]
    repeated = np.concatenate([d, d[:P]])
    bad = {"not whole pages": d[:-1], "misaligned page": d + 1, "out of range": d + g.device_slots,
           "rows out of order": swapped, "repeated page": repeated, "negative": d - P * 20}
    for what, lst in bad.items():
        try:
            O.layer_pack(g, 0, dev, lst)
        except ValueError:
            pass
        else:
            raise AssertionError(f"exchange accepted a bad list: {what}")
        try:
            O.layer_unpack(g, 0, dev, lst, np.zeros(max(O.layer_packed_bytes(g, P * 4), 1), np.uint8))
        except ValueError:
            pass
        else:
            raise AssertionError(f"unpack accepted a bad list: {what}")
    tok = GEOMS["pf_kv"]
    dev = random_device(tok, np.random.default_rng(991))
    assert O.layer_pack(tok, 0, dev, np.array([7, 3, 60, 11, 0])).size == 5 * (32 + 32)
    try:
        O.layer_pack(tok, 0, dev, np.array([7, 3, 7]))
    except ValueError:
        pass
    else:
        raise AssertionError("exchange accepted a repeated slot")


# ---------------------------------------------------------------- helpers the GPU tests rely on
def _refused(fn) -> bool:
    try:
        fn()
    except ValueError:
        return True
    return False


def pin_host_offsets_walk():
    """orc_host_offsets, the batched lookup with which the full-size GPU tests find the
    host bytes of every named row, against the structural walk's running sums: every host
    token of every geometry, in order and shuffled, for every sub-buffer and layer (a page
    block at every row of its page).  A token past the pool, a negative token, a bad
    sub-buffer or a bad layer is refused; an empty list gives no offsets."""
    for k, (name, g) in enumerate(GEOMS.items()):
        pos, _ = positions(g)
        P = g.page_size
        tokens = np.arange(g.host_pages * P, dtype=np.int64)
        shuffled = np.random.default_rng(1000 + k).permutation(tokens)
        for b, (gran, _) in enumerate(g.subs):
            for l in range(g.layers):
                for order in (tokens, shuffled):
                    if gran == B:
                        want = [pos[("blk", b, int(t) // P, l)][0] for t in order]
                    else:
                        want = [pos[("row", b, int(t) // P, l, int(t) % P)][0] for t in order]
                    got = O.host_offsets(g, b, l, order)
                    assert np.array_equal(got, np.array(want, dtype=np.int64)), (name, b, l)
        past = g.host_pages * P
        for bad in ([past], [-1], [0, 1, past]):
            assert _refused(lambda: O.host_offsets(g, 0, 0, bad)), (name, "token outside the pool accepted", bad)
        assert _refused(lambda: O.host_offsets(g, len(g.subs), 0, [0])), (name, "sub-buffer past the last accepted")
        assert _refused(lambda: O.host_offsets(g, -1, 0, [0])), (name, "negative sub-buffer accepted")
        assert _refused(lambda: O.host_offsets(g, 0, g.layers, [0])), (name, "layer past the last accepted")
        assert _refused(lambda: O.host_offsets(g, 0, -1, [0])), (name, "negative layer accepted")
        assert O.host_offsets(g, 0, 0, np.zeros(0, np.int64)).size == 0


def pin_host_offsets_golden():
    """The batched lookup at the workloads' full sizes (offsets far past 2^32) against the
    hand-derived closed forms: every host_offset line of the golden file, asked as the host
    token page * P + row."""
    with open(GOLDEN) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    seen = 0
    for ln in lines:
        name, geo, q = [x.strip() for x in ln.split("|")]
        lhs, rhs = [x.strip() for x in q.split("=")]
        what, *args = lhs.split()
        if what != "host_offset":
            continue
        layout, L, P, H, S, align, subs = geo.split()
        sub = [((T if s[0] == "T" else B), int(s[1:])) for s in subs.split(",")]
        lay = {"shard": O.KV_SPLIT_SHARD, "page_first": O.PAGE_FIRST, "token_major": O.PAGE_FIRST_TOKEN_MAJOR}[layout]
        g = O.Geometry(int(L), int(P), sub, int(H), int(S), lay, int(align))
        b, page, layer, row = [int(a) for a in args]
        got = O.host_offsets(g, b, layer, [page * int(P) + row])
        assert int(got[0]) == int(rhs), f"{name}: batched {lhs} = {int(got[0])}, closed form {rhs}"
        seen += 1
    assert seen >= 10


def _raw_geom(g: O.Geometry, nsub: int, tail: bytes = b"") -> ctypes.Array:
    """The C struct of g with its sub-buffer count overwritten, followed by `tail`: a way to
    hand the oracle a count its arrays cannot hold, with readable memory behind them."""
    c = g.c()
    c.nsub = nsub
    raw = bytes(c) + tail
    return (ctypes.c_uint8 * len(raw)).from_buffer_copy(raw)


def pin_geometry_refusals():
    """orc_check_geom, which every oracle entry point runs first: every geometry of these
    pins is accepted, and each rule refuses its own violation while a neighbour that keeps
    the rule is accepted.  Refused: zero layers, page size or sizes; no sub-buffer or more
    than four; an unknown layout or granularity; a shard layout with alignment 0 or
    negative; page blocks over a slot count that is not whole pages (token rows alone take
    any slot count)."""
    for name, g in GEOMS.items():
        assert O.check_geom(g), (name, "a pinned geometry refused")
    base = GEOMS["pf_kv"]
    def with_(**kw):
        d = dict(layers=base.layers, page_size=base.page_size, subs=list(base.subs), host_pages=base.host_pages,
                 device_slots=base.device_slots, layout=base.layout, align=base.align)
        d.update(kw)
        return O.Geometry(**d)
    for what, g in {"zero layers": with_(layers=0), "zero page size": with_(page_size=0),
                    "zero host pages": with_(host_pages=0), "zero device slots": with_(device_slots=0),
                    "no sub-buffer": with_(subs=[]), "unknown layout": with_(layout=3),
                    "zero row bytes": with_(subs=[(T, 32), (T, 0)]),
                    "unknown granularity": with_(subs=[(T, 32), (2, 32)]),
                    "shard alignment 0": with_(layout=O.KV_SPLIT_SHARD, align=0),
                    "negative shard alignment": with_(layout=O.KV_SPLIT_SHARD, align=-4096),
                    "page blocks over a partial device page": with_(subs=[(T, 32), (B, 48)], device_slots=65)}.items():
        assert not O.check_geom(g), f"oracle accepted a geometry with {what}"
    for what, g in {"four sub-buffers": with_(subs=[(T, 32)] * 4),
                    "shard alignment 16": with_(layout=O.KV_SPLIT_SHARD, align=16),
                    "token rows over 65 slots": with_(device_slots=65),
                    "page blocks over 64 slots": with_(subs=[(T, 32), (B, 48)], device_slots=64)}.items():
        assert O.check_geom(g), f"oracle refused a valid geometry with {what}"
    # Five sub-buffers: the struct holds four.  The oracle must refuse on the count alone,
    # so the memory a fifth entry would occupy is made to look valid: the fifth granularity
    # overlaps the low word of the first row size (2^32 + 0: token rows), the fifth size
    # sits right after the struct (16 bytes).
    four = with_(subs=[(T, (1 << 32)), (T, 32), (T, 32), (T, 32)])
    assert O.check_geom(four)
    raw = _raw_geom(four, 5, tail=(16).to_bytes(8, "little") * 4)
    lib = O.lib()
    assert lib.orc_check_geom(ctypes.cast(raw, ctypes.POINTER(O._Geom))) != 0, "oracle accepted five sub-buffers"
    # a refused geometry is refused by the entry points too
    assert _refused(lambda: O.host_offsets(with_(layout=O.KV_SPLIT_SHARD, align=0), 0, 0, [0]))


PINS = [pin_sizes_match_structure, pin_offsets_match_structure, pin_write_back_brute_force,
        pin_write_back_mock_formula, pin_load_back_brute_force, pin_round_trip_restores,
        pin_untouched_and_byte_accounting, pin_round_trip_check_counts, pin_index_preconditions,
        pin_golden_closed_forms, pin_h2h_shard_dump_and_load, pin_burst_algebra,
        pin_layer_exchange_gather_formula, pin_layer_exchange_restores_owner_rows, pin_layer_exchange_preconditions,
        pin_host_offsets_walk, pin_host_offsets_golden, pin_geometry_refusals]


def run_all() -> list:
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError as e:
            failed.append(f"{pin.__name__}: {e}")
    return failed


if __name__ == "__main__":
    bad = run_all()
    for b in bad:
        print("FAIL", b)
    sys.exit(1 if bad else 0)
