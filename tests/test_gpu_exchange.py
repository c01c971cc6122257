"""Per-layer exchange of a layer-owner sharded host tier, on one GPU (rank-sharded tier
page, sglang PR 41984, Modifications and Accuracy Tests).

Each host layer has one owner rank; after the owner has loaded a layer it packs the
rows into a staging buffer, the buffer goes to the other TP ranks, and they unpack it
into the same device slots.  Here the ranks' replicated device pools sit on one GPU
and the receiving rank reads the owner's staging buffer in place, standing in for the
broadcast (the collective itself needs more than one GPU).  Pack and unpack are checked
against the oracle byte for byte at the workloads' full per-layer sizes, and the whole
sharded load-back is checked end to end: every replica must equal the oracle's
load-back of the unsharded pool, and a skipped exchange (the page's negative control)
must show."""
import ctypes

import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import assert_bytes_equal, assert_dev_equal, cuda_i64, say, units
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def device_pool(shape, layers, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return [torch.empty((layers, units(shape, b) * e), dtype=torch.uint8, device="cuda").random_(0, 256, generator=gen)
            for b, (_, e) in enumerate(shape.subs)]


def device_only_pool(shape, layers, dev, stream, flags=0):
    """A pool with no host pages: the exchange and the round-trip check only."""
    return B.Pool(layers=layers, page_size=shape.page_size, subs=list(shape.subs), device_slots=shape.device_slots,
                  host_pages=0, device_layers=[[dev[b][l] for l in range(layers)] for b in range(len(shape.subs))],
                  host=None, stream=stream, flags=flags)


def oracle_geom(shape, layers, host_pages=1):
    return O.Geometry(layers, shape.page_size, [tuple(s) for s in shape.subs], host_pages, shape.device_slots,
                      shape.layout, shape.align)


def to_np(dev):
    return [[t[l].cpu().numpy() for l in range(t.shape[0])] for t in dev]


# Full-size per-layer bursts of every workload (the slots each draws), two layers of each pool.
FULL = ["tiny_mha_bf16", "llama3_8b_mha_bf16", "dsv3_mla_bf16", "dsa_mla_indexer_78l", "mha_kv_split_shard_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_pack_then_unpack_match_oracle(name):
    shape = W.SHAPES[name]
    L = 2
    burst = W.burst_for(shape, 71)
    d = burst.device_idx
    say(f"[exchange] {name} n={d.size} pack + unpack, layer 1")
    g = oracle_geom(shape, L)
    stream = torch.cuda.Stream()
    owner, other = device_pool(shape, L, 72), device_pool(shape, L, 73)
    torch.cuda.synchronize()
    owner0, other0 = to_np(owner), to_np(other)
    po, pr = device_only_pool(shape, L, owner, stream), device_only_pool(shape, L, other, stream)
    try:
        need = po.layer_pack_bytes(d.size)
        assert need == O.layer_packed_bytes(g, d.size)
        staging = torch.full((need + 64,), 0x5A, dtype=torch.uint8, device="cuda")
        d_t = cuda_i64(d)
        done = B.HipEvent()
        po.layer_pack(1, d_t, staging, done)
        pr.layer_unpack(1, staging, d_t, done)
        done.synchronize()
        po.sync()
        pr.sync()
        got = staging.cpu().numpy()
        assert_bytes_equal(got[:need], O.layer_pack(g, 1, owner0, d), "staging after pack")
        assert np.all(got[need:] == 0x5A), "pack wrote past its bytes"
        assert_dev_equal(to_np(owner), owner0, "pack changed the owner's pool")
        want = [[a.copy() for a in row] for row in other0]
        O.layer_unpack(g, 1, want, d, got[:need].copy())
        assert_dev_equal(to_np(other), want, "receiving pool after unpack")
    finally:
        po.close()
        pr.close()
        torch.cuda.synchronize()


@pytest.mark.parametrize("n", [0, 1, 17, 255, 257, 1000, 4096])
def test_ragged_token_lists(n):
    shape = W.SHAPES["tiny_mha_bf16"]
    L = 3
    d = W.permutation_slots(80 + n, shape.device_slots, n)
    g = oracle_geom(shape, L)
    stream = torch.cuda.Stream()
    owner, other = device_pool(shape, L, 81), device_pool(shape, L, 82)
    torch.cuda.synchronize()
    owner0, other0 = to_np(owner), to_np(other)
    po, pr = device_only_pool(shape, L, owner, stream), device_only_pool(shape, L, other, stream)
    try:
        staging = torch.zeros(max(po.layer_pack_bytes(n), 16), dtype=torch.uint8, device="cuda")
        d_t = cuda_i64(d)
        ev = B.HipEvent()
        po.layer_pack(2, d_t, staging, ev)
        pr.layer_unpack(2, staging, d_t, ev)
        ev.synchronize()
        assert ev.query()
        pr.sync()
        want = [[a.copy() for a in row] for row in other0]
        if n:
            packed = O.layer_pack(g, 2, owner0, d)
            assert_bytes_equal(staging.cpu().numpy()[:packed.size], packed, f"staging n={n}")
            O.layer_unpack(g, 2, want, d, packed)
        assert_dev_equal(to_np(other), want, f"receiving pool n={n}")
    finally:
        po.close()
        pr.close()
        torch.cuda.synchronize()


SHARDED = [
    # pool, layers, tp, device slots, host pages, burst pages
    ("dsa_mla_indexer_78l", 7, 3, 65536, 160, 64),
    ("dsv3_mla_bf16", 6, 2, 65536, 160, 48),
    ("llama3_8b_mha_bf16", 5, 4, 32768, 96, 40),
]


def run_sharded(case, skip_layer=None):
    """Sharded write-back then sharded load-back with the per-layer exchange; returns the
    ranks' device pools (numpy) and the oracle's unsharded result."""
    name, L, tp, S, H, npages = case
    base = W.shape_scaled(W.SHAPES[name], name, layers=L, device_slots=S, host_pages=H)
    P = base.page_size
    pages = W.host_pages(90, H, npages)
    h = W.whole_page_tokens(pages, P)
    blocks = any(gr == W.PAGE_BLOCKS for gr, _ in base.subs)
    d = W.page_aligned_slots(91, S, P, npages) if blocks else W.segment_slots(91, S, h.size)
    d2 = (W.page_aligned_slots(92, S, P, npages, exclude_pages=np.unique(d // P)) if blocks
          else W.segment_slots(92, S, h.size, exclude=d))
    full = device_pool(base, L, 93)
    torch.cuda.synchronize()
    full0 = to_np(full)
    ranks = []
    for r in range(tp):
        owned = list(range(r, L, tp))
        dev = [t.clone() for t in full]  # every rank holds the same device pool
        gr = oracle_geom(base, len(owned), H)
        host = B.HostBuffer(O.host_pool_bytes(gr))
        host.fill(0)
        stream = torch.cuda.Stream()
        share = B.Pool(layers=len(owned), page_size=P, subs=list(base.subs), device_slots=S, host_pages=H,
                       device_layers=[[dev[b][l] for l in owned] for b in range(len(base.subs))], host=host,
                       stream=stream)
        ranks.append(dict(owned=owned, dev=dev, host=host, stream=stream, share=share,
                          xpool=device_only_pool(base, L, dev, stream), geom=gr))
    try:
        torch.cuda.synchronize()
        h_np, d_t, h_t, d2_t = np.ascontiguousarray(h), cuda_i64(d), cuda_i64(h), cuda_i64(d2)
        for rk in ranks:  # each rank writes back only the layers it owns
            rk["share"].write_back_all_layers(d_t, h_np)
        for r, rk in enumerate(ranks):
            rk["share"].sync()
            want_host = np.zeros(rk["host"].nbytes, np.uint8)
            O.write_back(rk["geom"], [[full0[b][l] for l in rk["owned"]] for b in range(len(base.subs))], want_host,
                         d, h)
            assert_bytes_equal(rk["host"].np, want_host, f"rank {r} host pool after its write-back")
        staging = torch.empty((L, ranks[0]["xpool"].layer_pack_bytes(h.size)), dtype=torch.uint8, device="cuda")
        layer_done = [[B.HipEvent() for _ in range(L)] for _ in ranks]
        for l in range(L):
            owner = ranks[l % tp]
            owner["share"].load_back_layer(l // tp, h_t, d2_t)
            packed = layer_done[l % tp][l]  # the owner's layer is done once its exchange is out
            owner["xpool"].layer_pack(l, d2_t, staging[l], packed)
            for q, rk in enumerate(ranks):
                if q == l % tp or (skip_layer == l and q == (l + 1) % tp):
                    continue
                packed.wait_on(rk["stream"])
                rk["xpool"].layer_unpack(l, staging[l], d2_t, layer_done[q][l])
        for evs in layer_done:
            for ev in evs:
                ev.synchronize()
        torch.cuda.synchronize()
        for rk in ranks:
            rk["share"].sync()
            rk["xpool"].sync()
        # the oracle's unsharded pool: every layer written back to one host pool, loaded into d2
        g = oracle_geom(base, L, H)
        host_full = np.zeros(O.host_pool_bytes(g), np.uint8)
        O.write_back(g, full0, host_full, d, h)
        want = [[a.copy() for a in row] for row in full0]
        for l in range(L):
            O.load_back_layer(g, l, want, host_full, h, d2)
        return [to_np(rk["dev"]) for rk in ranks], want
    finally:
        for rk in ranks:
            rk["xpool"].close()
            rk["share"].close()
            rk["host"].free()
        torch.cuda.synchronize()


@pytest.mark.parametrize("case", SHARDED, ids=[f"{c[0]}_tp{c[2]}" for c in SHARDED])
def test_sharded_load_back_restores_every_replica(case):
    say(f"[exchange] sharded round trip {case}")
    replicas, want = run_sharded(case)
    for r, dev in enumerate(replicas):
        assert_dev_equal(dev, want, f"rank {r} device pool")


def test_skipped_exchange_is_caught():
    case = SHARDED[1]
    say(f"[exchange] negative control {case}")
    replicas, want = run_sharded(case, skip_layer=3)
    tp = case[2]
    bad = (3 + 1) % tp
    for r, dev in enumerate(replicas):
        if r != bad:
            assert_dev_equal(dev, want, f"rank {r} device pool")
    with pytest.raises(AssertionError):
        assert_dev_equal(replicas[bad], want, "the rank that skipped the exchange of layer 3")


def test_refusals_and_device_reports():
    shape = W.shape_scaled(W.SHAPES["dsa_mla_indexer_78l"], "x", layers=2, device_slots=8192, host_pages=8)
    P, S = shape.page_size, shape.device_slots
    stream = torch.cuda.Stream()
    dev = device_pool(shape, 2, 95)
    torch.cuda.synchronize()
    pool = device_only_pool(shape, 2, dev, stream)
    checked = device_only_pool(shape, 2, dev, stream, flags=B.HC_FLAG_VALIDATE)
    host = B.HostBuffer(1 << 20)
    try:
        d = W.page_aligned_slots(96, S, P, 3, exclude_pages=np.array([S // P - 1]))  # room to shift a page by one
        d_t = cuda_i64(d)
        need = pool.layer_pack_bytes(d.size)
        staging = torch.zeros(need + 64, dtype=torch.uint8, device="cuda")
        # a device-only pool refuses host transfers, and still records the event
        ev = B.HipEvent()
        with pytest.raises(B.HcError) as e:
            pool.write_back_all_layers(d_t, np.ascontiguousarray(d), ev)
        assert e.value.code == B.HC_ERR_INVALID and "no host pages" in str(e.value)
        ev.synchronize()
        with pytest.raises(B.HcError) as e:
            pool.load_back_layer(0, d_t, d_t, ev)
        assert e.value.code == B.HC_ERR_INVALID and "no host pages" in str(e.value)
        with pytest.raises(B.HcError):
            pool.capture_load_back(d_t, d_t, [None, None])
        with pytest.raises(B.HcError):
            B.Loader(pool, 2)
        # staging too small, misaligned, host memory; whole pages; layer range
        with pytest.raises(B.HcError) as e:
            pool.layer_pack(0, d_t, staging[:need - 16])
        assert e.value.code == B.HC_ERR_INVALID
        with pytest.raises(B.HcError) as e:
            pool.layer_pack(0, d_t, staging[8:8 + need])
        assert e.value.code == B.HC_ERR_UNSUPPORTED
        rc = B.lib.hc_layer_pack(pool.handle, 0, B._V(d_t.data_ptr()), d.size, B._V(host.ptr.value), host.nbytes,
                                 None)
        assert rc == B.HC_ERR_INVALID and b"device memory" in B.lib.hc_last_error()
        with pytest.raises(B.HcError):
            pool.layer_pack(0, d_t[:P + 1], staging)
        with pytest.raises(B.HcError) as e:
            pool.layer_unpack(2, staging, d_t, ev)
        assert e.value.code == B.HC_ERR_INVALID
        ev.synchronize()
        with pytest.raises(B.HcError):
            pool.layer_pack_bytes(P - 1)
        pool.sync()
        # an out-of-range slot is skipped and reported with its list position
        bad = d.copy()
        bad[P + 5] = S + 3  # a latent row; the page's indexer block is taken at position P
        pool.layer_unpack(1, staging, cuda_i64(bad), ev)
        ev.synchronize()
        with pytest.raises(B.HcError) as e:
            pool.sync()
        assert e.value.code == B.HC_ERR_DEVICE and f"first flagged list position {P + 5})" in str(e.value)
        # with HC_FLAG_VALIDATE a page-block page must be one whole device page
        shifted = d.copy()
        shifted[P:2 * P] += 1
        assert shifted.max() < S
        pool.layer_pack(1, cuda_i64(shifted), staging)
        pool.sync()  # without HC_FLAG_VALIDATE the page's shape is trusted
        checked.layer_pack(1, cuda_i64(shifted), staging)
        with pytest.raises(B.HcError) as e:
            checked.sync()
        assert e.value.code == B.HC_ERR_DEVICE and "page-block" in str(e.value)
        assert f"first flagged list position {P})" in str(e.value), str(e.value)
        checked.sync()  # cleared once reported
        checked.layer_pack(1, d_t, staging)
        checked.sync()
    finally:
        checked.close()
        pool.close()
        host.free()
        torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(200))
def test_random_exchange(seed):
    """Random pools of the randomized parity sweep (layers, page size, row and block sizes,
    partial pages, slot patterns): one random layer packed and unpacked against the oracle."""
    from test_gpu_random import random_case
    shape, d, _h, _d2, _mode, _staging, _ctas = random_case(seed)
    rng = np.random.default_rng(7000 + seed)
    L = shape.layers
    layer = int(rng.integers(0, L))
    flags = B.HC_FLAG_VALIDATE if rng.random() < 0.3 else 0
    say(f"[exchange random {seed}] L={L} P={shape.page_size} subs={shape.subs} n={d.size} layer={layer} flags={flags}")
    g = oracle_geom(shape, L)
    stream = torch.cuda.Stream()
    owner, other = device_pool(shape, L, 7100 + seed), device_pool(shape, L, 7200 + seed)
    torch.cuda.synchronize()
    owner0, other0 = to_np(owner), to_np(other)
    po = device_only_pool(shape, L, owner, stream, flags=flags)
    pr = device_only_pool(shape, L, other, stream, flags=flags)
    try:
        need = po.layer_pack_bytes(d.size)
        staging = torch.full((need + 16,), 0xC3, dtype=torch.uint8, device="cuda")
        d_t = cuda_i64(d)
        po.layer_pack(layer, d_t, staging)
        pr.layer_unpack(layer, staging, d_t)
        po.sync()
        pr.sync()
        got = staging.cpu().numpy()
        packed = O.layer_pack(g, layer, owner0, d)
        assert_bytes_equal(got[:need], packed, "staging after pack")
        assert np.all(got[need:] == 0xC3), "pack wrote past its bytes"
        want = [[a.copy() for a in row] for row in other0]
        O.layer_unpack(g, layer, want, d, packed)
        assert_dev_equal(to_np(other), want, "receiving pool after unpack")
        assert_dev_equal(to_np(owner), owner0, "pack changed the owner's pool")
    finally:
        po.close()
        pr.close()


def test_exchange_in_a_captured_graph():
    """Pack and unpack captured into a HIP graph on the pools' stream (a caller that replays
    its per-layer exchange instead of enqueueing it), replayed three times with eager
    writes to the owner's layer in between; every replay is checked against the oracle."""
    shape = W.SHAPES["dsa_mla_indexer_78l"]
    shape = W.shape_scaled(shape, "graph", layers=3, device_slots=65536, host_pages=8)
    L = shape.layers
    d = W.page_aligned_slots(120, shape.device_slots, shape.page_size, 40)
    g = oracle_geom(shape, L)
    stream = torch.cuda.Stream()
    owner, other = device_pool(shape, L, 121), device_pool(shape, L, 122)
    po, pr = device_only_pool(shape, L, owner, stream), device_only_pool(shape, L, other, stream)
    try:
        d_t = cuda_i64(d)
        staging = torch.zeros(po.layer_pack_bytes(d.size), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream, capture_error_mode="thread_local"):
            po.layer_pack(1, d_t, staging)
            pr.layer_unpack(1, staging, d_t)
        torch.cuda.synchronize()
        gen = torch.Generator(device="cuda")
        gen.manual_seed(123)
        for replay in range(3):
            for t in owner:  # new rows to exchange, written eagerly between replays
                t[1].random_(0, 256, generator=gen)
            torch.cuda.synchronize()
            owner0, other0 = to_np(owner), to_np(other)
            graph.replay()
            torch.cuda.synchronize()
            po.sync()
            pr.sync()
            packed = O.layer_pack(g, 1, owner0, d)
            assert_bytes_equal(staging.cpu().numpy(), packed, f"staging after replay {replay}")
            want = [[a.copy() for a in row] for row in other0]
            O.layer_unpack(g, 1, want, d, packed)
            assert_dev_equal(to_np(other), want, f"receiving pool after replay {replay}")
        del graph
    finally:
        po.close()
        pr.close()
        torch.cuda.synchronize()
