"""One rank's share of a layer-owner sharded host tier (rank-sharded tier page,
Modifications): rank r of tp owns the layers l with l % tp == r and moves only those.
On one GPU the share is a pool over the owned layers' device buffers (the pool takes
one pointer per layer), with a host pool of the owned layers only.  Checked against the
oracle on the owned layers' geometry; the layers the rank does not own stay untouched."""
import numpy as np
import pytest
import torch

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import assert_bytes_equal, cuda_i64, say
from oracle import oracle as O

T, BLK = W.TOKEN_ROWS, W.PAGE_BLOCKS

CASES = [
    # name, layers, tp, rank, page size, sub-buffers, device slots, host pages
    ("mla_latent_tp4_rank1", 10, 4, 1, 64, ((T, 1152),), 16384, 48),
    ("mla_indexer_tp3_rank2", 7, 3, 2, 64, ((T, 1152), (BLK, 8448)), 8192, 24),
]


@pytest.mark.gpu
@pytest.mark.parametrize("staged", [False, True], ids=["zerocopy", "staged"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rank_share_moves_only_owned_layers(case, staged):
    name, L, tp, rank, P, subs, S, H = case
    owned = list(range(rank, L, tp))
    say(f"[rank share] {name} owned layers {owned} staged={staged}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    dev = []  # the full device pool: every layer, as on every TP rank
    for g, e in subs:
        units = S // P if g == BLK else S
        dev.append(torch.empty((L, units * e), dtype=torch.uint8, device="cuda").random_(0, 256, generator=gen))
    geom = O.Geometry(len(owned), P, [tuple(s) for s in subs], H, S, W.PAGE_FIRST, 4096)
    host = B.HostBuffer(O.host_pool_bytes(geom))
    host.np[:] = np.random.default_rng(32).integers(0, 256, host.np.size, dtype=np.uint8)
    staging = None
    if staged:
        img = O.page_payload_bytes(geom)
        staging = torch.empty(3 * img, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    pool = B.Pool(layers=len(owned), page_size=P, subs=list(subs), device_slots=S, host_pages=H,
                  device_layers=[[dev[b][l] for l in owned] for b in range(len(subs))], host=host, stream=stream,
                  staging=staging,
                  write_back_mode=B.HC_MODE_STAGED if staged else B.HC_MODE_ZEROCOPY)
    try:
        pages = W.host_pages(33, H, 9)
        h = W.whole_page_tokens(pages, P)
        d = W.page_aligned_slots(34, S, P, pages.size)
        d2 = W.page_aligned_slots(35, S, P, pages.size, exclude_pages=np.unique(d // P))
        torch.cuda.synchronize()
        full0 = [t.cpu().numpy() for t in dev]
        host0 = host.np.copy()
        # write-back of the owned layers
        pool.write_back_all_layers(cuda_i64(d), h)
        pool.sync()
        want_host = host0.copy()
        own_dev = [[full0[b][l] for l in owned] for b in range(len(subs))]
        O.write_back(geom, own_dev, want_host, d, h)
        assert_bytes_equal(host.np, want_host, "rank host pool after write-back")
        # per-layer load-back of the owned layers into fresh slots (owned layer k = model layer owned[k])
        for k in range(len(owned)):
            pool.load_back_layer(k, cuda_i64(h), cuda_i64(d2))
        pool.sync()
        want = [[a.copy() for a in row] for row in own_dev]
        for k in range(len(owned)):
            O.load_back_layer(geom, k, want, want_host, h, d2)
        for b in range(len(subs)):
            got = dev[b].cpu().numpy()
            for l in range(L):
                expect = want[b][owned.index(l)] if l in owned else full0[b][l]
                assert_bytes_equal(got[l], expect, f"sub {b} model layer {l} ({'owned' if l in owned else 'not owned'})")
    finally:
        pool.close()
        host.free()
        torch.cuda.synchronize()
