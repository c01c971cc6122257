"""GPU path vs oracle, bit-exact, at sizes the oracle finishes in seconds.

Each case spans several 256-token tiles with a ragged tail, and compares the
whole host pool after write-back and the whole device pool after per-layer
load-back with the oracle run on the same seeded inputs.  Modes: zero-copy and
staged (staging chunks smaller than the burst, so several chunks run)."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, load_back_and_check, say, write_back_and_check

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS
PF, SH, TM = W.PAGE_FIRST, W.KV_SPLIT_SHARD, W.PAGE_FIRST_TOKEN_MAJOR


def S(name, L, P, subs, slots, pages, layout=PF, align=4096):
    return W.PoolShape(name, L, P, tuple(subs), slots, pages, layout, align)


def has_blocks(shape):
    return any(g == BLK for g, _ in shape.subs)


def burst(shape, seed, kind, pages, partial_rows=0):
    """(device slots, host tokens) for a case.
    kind: 'perm' random distinct slots, 'segment' free-list runs, 'aligned' whole device pages,
    'scatter' no adjacent neighbours, 'requests' partial-page requests."""
    P = shape.page_size
    if kind == "requests":
        h = W.partial_page_requests(seed, shape.host_pages, P, pages)
    else:
        pg = W.host_pages(seed, shape.host_pages, pages)
        h = W.whole_page_tokens(pg, P)
        if partial_rows:
            extra = np.setdiff1d(np.arange(shape.host_pages), pg)[0]
            h = np.concatenate([h, extra * P + np.arange(partial_rows)])
    n = h.size
    if kind == "aligned":
        d = W.page_aligned_slots(seed + 1, shape.device_slots, P, n // P)
    elif kind == "segment":
        d = W.segment_slots(seed + 1, shape.device_slots, n)
    elif kind == "scatter":
        d = W.scattered_slots(seed + 1, shape.device_slots, n)
    else:
        d = W.permutation_slots(seed + 1, shape.device_slots, n)
    return d, h


def fresh(shape, d, seed):
    P = shape.page_size
    if has_blocks(shape):
        return W.page_aligned_slots(seed, shape.device_slots, P, d.size // P, exclude_pages=np.unique(d // P))
    return W.permutation_slots(seed, shape.device_slots, d.size, exclude=d)


CASES = [
    # name, shape, burst kind, pages, partial rows
    ("tiny_mha_bf16", W.SHAPES["tiny_mha_bf16"], "perm", 32, 0),
    ("llama_rows_small", S("llama_rows_small", 4, 64, [(T, 2048)] * 2, 32768, 64), "segment", 12, 41),
    ("mla_latent_small", S("mla_latent_small", 3, 64, [(T, 1152)], 65536, 64), "segment", 9, 17),
    ("mla_indexer_small", S("mla_indexer_small", 3, 64, [(T, 1152), (BLK, 8448)], 8192, 32), "aligned", 10, 0),
    ("shard_kv_small", S("shard_kv_small", 4, 32, [(T, 2048)] * 2, 16384, 64, SH), "requests", 24, 0),
    ("shard_kv_pad", S("shard_kv_pad", 3, 16, [(T, 1024), (T, 128)], 4096, 40, SH), "requests", 30, 0),
    ("elem16_rows", S("elem16_rows", 2, 8, [(T, 16)], 4096, 64), "requests", 50, 0),
    ("elem_max_rows", S("elem_max_rows", 2, 4, [(T, 65536)], 64, 8), "perm", 3, 2),
    ("page1_rows", S("page1_rows", 3, 1, [(T, 32)], 2048, 1024), "scatter", 700, 0),
    ("four_subs_one_layer", S("four_subs_one_layer", 1, 16, [(T, 48), (T, 16), (BLK, 32), (T, 64)], 2048, 64),
     "aligned", 33, 0),
    ("token_major_rows", S("token_major_rows", 4, 64, [(T, 2048)] * 2, 32768, 64, TM), "segment", 12, 41),
    ("token_major_indexer", S("token_major_indexer", 3, 64, [(T, 1152), (BLK, 8448)], 8192, 32, TM), "aligned", 10, 0),
    ("token_major_small_rows", S("token_major_small_rows", 5, 8, [(T, 16), (T, 48)], 4096, 64, TM), "requests", 50, 0),
    # the largest layer count the descriptor accepts (HC_MAX_LAYERS), rows and page blocks
    ("max_layers", S("max_layers", 1024, 4, [(T, 16), (BLK, 32)], 256, 8), "aligned", 3, 0),
]


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["zerocopy", "staged"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_write_back_then_load_back(case, mode):
    name, shape, kind, pages, partial = case
    say(f"[parity] {name} mode={mode}")
    d, h = burst(shape, 11, kind, pages, partial)
    wb = B.HC_MODE_STAGED if mode == "staged" else B.HC_MODE_ZEROCOPY
    # staging smaller than the burst: several chunks
    rig = Rig(shape, seed=5, write_back_mode=wb, staging_pages=max(1, pages // 3) if mode == "staged" else 0)
    try:
        assert rig.pool.mode(0) == wb and rig.pool.mode(1) == B.HC_MODE_ZEROCOPY
        write_back_and_check(rig, d, h)
        d2 = fresh(shape, d, 23)
        load_back_and_check(rig, h, d2)
        assert rig.pool.round_trip_check(cuda_i64(d), cuda_i64(d2)) == 0
    finally:
        rig.close()


GRID_SHAPE = S("grid_small", 2, 4, [(T, 32)] * 2, 4096, 256)
GRID_SHARD = S("grid_shard", 2, 4, [(T, 32), (T, 16)], 4096, 256, SH, 256)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [GRID_SHAPE, GRID_SHARD], ids=lambda s: s.name)
@pytest.mark.parametrize("pages", [1, 63, 64, 65, 128, 129])
def test_staged_chunk_boundaries(shape, pages):
    """Page counts around one and two 64-page staging chunks."""
    say(f"[chunks] {shape.name} pages={pages}")
    d, h = burst(shape, pages, "perm", pages)
    rig = Rig(shape, seed=pages, write_back_mode=B.HC_MODE_STAGED, staging_pages=64)
    try:
        write_back_and_check(rig, d, h)
    finally:
        rig.close()


@pytest.mark.gpu
def test_staged_interleaved_pages():
    """Tokens of pages interleaved across chunks: split pages take the zero-copy path."""
    shape = GRID_SHAPE
    say("[interleaved] staged")
    pg = W.host_pages(3, shape.host_pages, 12)
    h = W.whole_page_tokens(pg, shape.page_size)
    rng = np.random.default_rng(4)
    h = h[rng.permutation(h.size)]
    d = W.permutation_slots(5, shape.device_slots, h.size)
    rig = Rig(shape, seed=9, write_back_mode=B.HC_MODE_STAGED, staging_pages=4)
    try:
        write_back_and_check(rig, d, h)
        load_back_and_check(rig, h, fresh(shape, d, 6))
    finally:
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [B.HC_MODE_ZEROCOPY, B.HC_MODE_STAGED])
def test_empty_and_single(mode):
    shape = GRID_SHAPE
    say(f"[edge] empty/single mode={mode}")
    rig = Rig(shape, seed=1, write_back_mode=mode, staging_pages=2)
    try:
        ev = B.HipEvent()
        e = torch.empty(0, dtype=torch.int64, device="cuda")
        rig.pool.write_back_all_layers(e, np.empty(0, dtype=np.int64), ev)
        ev.synchronize()
        rig.pool.load_back_layer(0, e, e, ev)
        ev.synchronize()
        assert rig.pool.round_trip_check(e, e) == 0
        # the last slot and the last host row
        last_d = np.array([shape.device_slots - 1])
        last_h = np.array([shape.host_pages * shape.page_size - 1])
        write_back_and_check(rig, last_d, last_h)
        load_back_and_check(rig, last_h, np.array([0]))
    finally:
        rig.close()


@pytest.mark.gpu
def test_validate_flag_accepts_whole_pages():
    shape = CASES[3][1]
    say("[validate] whole pages")
    d, h = burst(shape, 2, "aligned", 6)
    rig = Rig(shape, seed=2, flags=B.HC_FLAG_VALIDATE)
    try:
        write_back_and_check(rig, d, h)
        load_back_and_check(rig, h, fresh(shape, d, 3))
    finally:
        rig.close()


# Small bursts on grids of 1 to 256 workgroups: the zero-copy kernels shrink their token
# tile (down to 4 tokens) until the burst gives every workgroup a unit.  Token rows of
# several sizes, page blocks that only the tile holding a page's row 0 moves, shards.
SPLIT_SHAPES = [
    S("split_rows_kv", 3, 16, [(T, 2048)] * 2, 8192, 64),
    S("split_latent_indexer", 2, 16, [(T, 1152), (BLK, 8448)], 4096, 32),
    S("split_odd_rows", 2, 8, [(T, 48), (T, 2048)], 4096, 64),
    S("split_shard", 2, 8, [(T, 1024), (T, 128)], 4096, 64, SH),
]


@pytest.mark.gpu
@pytest.mark.parametrize("max_ctas", [1, 16, 64, 256])
@pytest.mark.parametrize("pages", [1, 3, 20])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: s.name)
def test_small_bursts_shrink_tiles(shape, pages, max_ctas):
    """Bursts too small to fill the grid run on shrunk tiles; results stay bit-exact."""
    say(f"[small] {shape.name} pages={pages} max_ctas={max_ctas}")
    kind = "aligned" if has_blocks(shape) else ("requests" if shape.layout == SH else "perm")
    d, h = burst(shape, pages, kind, pages)
    rig = Rig(shape, seed=pages, max_ctas=max_ctas)
    try:
        write_back_and_check(rig, d, h)
        load_back_and_check(rig, h, fresh(shape, d, pages + 7))
    finally:
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("staging_pages,want", [(0, B.HC_MODE_ZEROCOPY), (2, B.HC_MODE_STAGED)])
def test_auto_mode_stages_write_back_when_staging_is_given(staging_pages, want):
    """HC_MODE_AUTO: staged write-back with a staging buffer, zero-copy without; both bit-exact."""
    shape = GRID_SHAPE
    say(f"[auto] staging_pages={staging_pages}")
    d, h = burst(shape, 3, "perm", 9)
    rig = Rig(shape, seed=3, write_back_mode=B.HC_MODE_AUTO, staging_pages=staging_pages)
    try:
        assert rig.pool.mode(0) == want and rig.pool.mode(1) == B.HC_MODE_ZEROCOPY
        write_back_and_check(rig, d, h)
        load_back_and_check(rig, h, fresh(shape, d, 4))
    finally:
        rig.close()


# A chunk's last whole page and the next chunk's first whole page sit in consecutive
# staging slots and on consecutive host pages, with partly named pages between them:
# their copy-engine regions are adjacent on both sides but must stay separate, because
# the second page's image is gathered only with the second chunk.
MERGE_SHAPES = [
    S("merge_shards", 2, 8, [(T, 64), (T, 64)], 4096, 32, SH, 256),
    S("merge_shards_pad", 2, 8, [(T, 64), (T, 48)], 4096, 32, SH, 4096),
    S("merge_one_sub", 2, 8, [(T, 64)], 4096, 32),
]


@pytest.mark.gpu
@pytest.mark.parametrize("shape", MERGE_SHAPES, ids=lambda s: s.name)
def test_staged_regions_stay_inside_their_chunk(shape):
    say(f"[chunks] adjacent regions across chunks {shape.name}")
    P = shape.page_size
    whole = lambda p: list(range(p * P, (p + 1) * P))
    h = np.array(whole(5) + [20 * P + r for r in range(3)] + [9 * P + r for r in range(2)] + whole(6), dtype=np.int64)
    d = W.permutation_slots(3, shape.device_slots, h.size)
    rig = Rig(shape, seed=21, write_back_mode=B.HC_MODE_STAGED, staging_pages=2)
    try:
        for _ in range(2):  # the second burst finds the staging slots holding the first one's images
            write_back_and_check(rig, d, h)
            d = W.permutation_slots(4, shape.device_slots, h.size)
    finally:
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["zerocopy", "staged"])
def test_page_method_names(mode):
    """backup_from_device_all_layer / load_to_device_per_layer (the host-pool names of the
    pages, host indices first) move what the oracle moves."""
    from gpu_support import assert_bytes_equal, assert_dev_equal
    from oracle import oracle as O
    shape = W.SHAPES["tiny_mha_bf16"]
    say(f"[parity] page method names, {mode}")
    rig = Rig(shape, seed=41, staging_pages=3 if mode == "staged" else 0,
              write_back_mode=B.HC_MODE_STAGED if mode == "staged" else B.HC_MODE_ZEROCOPY)
    try:
        d, h = burst(shape, 42, "perm", 7, 5)
        dev0, host0 = rig.dev_np(), rig.host.np.copy()
        torch.cuda.synchronize()
        rig.pool.backup_from_device_all_layer(np.ascontiguousarray(h, dtype=np.int64), cuda_i64(d))
        rig.pool.sync()
        want_host = host0.copy()
        O.write_back(rig.geom, dev0, want_host, d, h)
        assert_bytes_equal(rig.host.np, want_host, "host pool after backup_from_device_all_layer")
        d2 = fresh(shape, d, 43)
        ev = B.HipEvent()
        for l in range(shape.layers):
            rig.pool.load_to_device_per_layer(cuda_i64(h), cuda_i64(d2), l, ev if l == shape.layers - 1 else None)
        ev.synchronize()
        rig.pool.sync()
        want = [[a.copy() for a in row] for row in dev0]
        for l in range(shape.layers):
            O.load_back_layer(rig.geom, l, want, want_host, h, d2)
        assert_dev_equal(rig.dev_np(), want, "device pool after load_to_device_per_layer")
    finally:
        rig.close()


@pytest.mark.gpu
def test_shard_pads_stay_zero_when_staging_is_shared():
    """A shard pool's staging images carry the zero pad of every whole shard they send.
    Another pool using the same staging buffer between its bursts (or anything else
    writing there) must not leak into the host shards' pads."""
    from gpu_support import assert_bytes_equal
    from oracle import oracle as O
    shape = S("shared_staging_pad", 3, 16, [(T, 1024), (T, 128)], 4096, 40, SH)
    other = S("shared_staging_rows", 2, 16, [(T, 4096)], 4096, 40)
    say("[parity] shard pads with a shared staging buffer")
    rig = Rig(shape, seed=51, staging_pages=3, write_back_mode=B.HC_MODE_STAGED)
    orig = Rig(other, seed=52, fill_device=True)
    opool = None
    try:
        # a page-first pool over other buffers, staged through the shard pool's staging buffer
        opool = B.Pool(layers=other.layers, page_size=other.page_size, subs=list(other.subs),
                       device_slots=other.device_slots, host_pages=other.host_pages,
                       device_layers=[[orig.dev[b][l] for l in range(other.layers)] for b in range(1)],
                       host=orig.host, stream=rig.stream, staging=rig.staging, write_back_mode=B.HC_MODE_STAGED)
        for r, scribble in enumerate(["none", "fill", "other pool"]):
            if scribble == "fill":
                rig.staging.fill_(0xEE)
            elif scribble == "other pool":
                pg = W.host_pages(60, other.host_pages, 5)
                oh = W.whole_page_tokens(pg, other.page_size)
                opool.write_back_all_layers(cuda_i64(W.permutation_slots(61, other.device_slots, oh.size)), oh)
                opool.sync()
            d, h = burst(shape, 70 + r, "perm", 7)
            dev0, host0 = rig.dev_np(), rig.host.np.copy()
            torch.cuda.synchronize()
            rig.pool.write_back_all_layers(cuda_i64(d), np.ascontiguousarray(h, dtype=np.int64))
            rig.pool.sync()
            want = host0.copy()
            O.write_back(rig.geom, dev0, want, d, h)
            assert_bytes_equal(rig.host.np, want, f"host shards after a write-back (staging scribbled: {scribble})")
    finally:
        if opool is not None:
            opool.close()
        orig.close()
        rig.close()


@pytest.mark.gpu
def test_pool_on_the_null_stream():
    """copy_stream NULL: the pool's work goes to the null stream; transfers still match the
    oracle, and capturing a graph there is refused with an error, not a crash."""
    from gpu_support import assert_bytes_equal, assert_dev_equal
    from oracle import oracle as O
    shape = W.SHAPES["tiny_mha_bf16"]
    say("[parity] pool on the null stream")
    rig = Rig(shape, seed=95)
    pool = None
    try:
        L = shape.layers
        pool = B.Pool(layers=L, page_size=shape.page_size, subs=list(shape.subs),
                      device_slots=shape.device_slots, host_pages=shape.host_pages,
                      device_layers=[[rig.dev[b][l] for l in range(L)] for b in range(len(shape.subs))],
                      host=rig.host, stream=None, write_back_mode=B.HC_MODE_ZEROCOPY)
        d, h = burst(shape, 96, "perm", 5, 3)
        dev0, host0 = rig.dev_np(), rig.host.np.copy()
        pool.write_back_all_layers(cuda_i64(d), h)
        d2 = fresh(shape, d, 97)
        for l in range(L):
            pool.load_back_layer(l, cuda_i64(h), cuda_i64(d2))
        pool.sync()
        want_host = host0.copy()
        O.write_back(rig.geom, dev0, want_host, d, h)
        for l in range(L):
            O.load_back_layer(rig.geom, l, dev0, want_host, h, d2)
        assert_bytes_equal(rig.host.np, want_host, "host pool")
        assert_dev_equal(rig.dev_np(), dev0, "device pool")
        with pytest.raises(B.HcError):
            pool.capture_load_back(cuda_i64(h), cuda_i64(d2), [B.HipEvent() for _ in range(L)])
        pool.load_back_layer(0, cuda_i64(h), cuda_i64(d2))  # still usable after the refused capture
        pool.sync()
    finally:
        if pool is not None:
            pool.close()
        rig.close()


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["torch_cpu", "torch_pinned"])
def test_write_back_host_list_as_a_torch_tensor(kind):
    """The write-back's host list may be a torch CPU tensor, pageable or pinned, as well as a
    numpy array."""
    from gpu_support import assert_bytes_equal
    from oracle import oracle as O
    shape = W.SHAPES["tiny_mha_bf16"]
    say(f"[parity] host list as {kind}")
    rig = Rig(shape, seed=98, staging_pages=2, write_back_mode=B.HC_MODE_STAGED)
    try:
        d, h = burst(shape, 99, "perm", 6, 4)
        h_t = torch.from_numpy(np.ascontiguousarray(h, dtype=np.int64))
        if kind == "torch_pinned":
            h_t = h_t.pin_memory()
        dev0, host0 = rig.dev_np(), rig.host.np.copy()
        torch.cuda.synchronize()
        rig.pool.write_back_all_layers(cuda_i64(d), h_t)
        rig.pool.sync()
        want = host0.copy()
        O.write_back(rig.geom, dev0, want, d, h)
        assert_bytes_equal(rig.host.np, want, "host pool")
    finally:
        rig.close()
