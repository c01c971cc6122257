"""One TP rank of a layer-owner sharded host tier (rank-sharded tier page, sglang PR 41984,
Modifications and Accuracy Tests), run as its own process by
tests/test_gpu_rank_shard_gloo.py.  Test infrastructure.

Every rank holds the same device pool (same seed) and owns the host layers l with
l % world == rank.  It writes back only its own layers; on load-back the owner of each
layer loads it, packs it (hc_layer_pack) and broadcasts the packed bytes over gloo, and
every other rank unpacks them into the same slots (hc_layer_unpack).  gloo carries CPU
tensors only, so the packed bytes go through host memory with synchronous copies; on a
multi-GPU node the same broadcast is RCCL over xGMI on device memory.

Each rank then checks its device pool against the oracle's unsharded load-back, and the
ranks compare a digest of their pools and a fingerprint of the host pages they loaded
(the page's periodic cross-rank check).  Environment: RANK, WORLD_SIZE, MASTER_ADDR,
MASTER_PORT; HC_DIVERGE_RANK makes that rank use other host pages, HC_SKIP_RANK makes
that rank skip its unpacks (the page's two negative controls).  Prints one JSON line."""
import datetime
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402
import torch  # noqa: E402
import torch.distributed as dist  # noqa: E402

from host_device_page_amd import binding as B  # noqa: E402
from host_device_page_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402

L, S, H, NPAGES = 7, 65536, 160, 48


def main():
    rank, world = int(os.environ["RANK"]), int(os.environ["WORLD_SIZE"])
    diverge, skip = int(os.environ.get("HC_DIVERGE_RANK", "-1")), int(os.environ.get("HC_SKIP_RANK", "-1"))
    # a rank that fails leaves the others in a collective: bounded, so they fail too
    dist.init_process_group("gloo", rank=rank, world_size=world, timeout=datetime.timedelta(seconds=90))
    torch.cuda.set_device(0)
    shape = W.shape_scaled(W.SHAPES["dsa_mla_indexer_78l"], "rank_shard", layers=L, device_slots=S, host_pages=H)
    P, subs = shape.page_size, list(shape.subs)
    # replicated state: the same device pool, host pages and slots on every rank
    gen = torch.Generator(device="cuda")
    gen.manual_seed(93)
    dev = [torch.empty((L, (S // P if g == W.PAGE_BLOCKS else S) * e), dtype=torch.uint8, device="cuda")
           .random_(0, 256, generator=gen) for g, e in subs]
    pages = W.host_pages(90 if rank != diverge else 190, H, NPAGES)
    h = W.whole_page_tokens(pages, P)
    d = W.page_aligned_slots(91, S, P, NPAGES)
    d2 = W.page_aligned_slots(92, S, P, NPAGES, exclude_pages=np.unique(d // P))
    torch.cuda.synchronize()
    full0 = [[t[l].cpu().numpy() for l in range(L)] for t in dev]

    owned = list(range(rank, L, world))
    geom_own = O.Geometry(len(owned), P, [tuple(s) for s in subs], H, S)
    host = B.HostBuffer(O.host_pool_bytes(geom_own))
    stream = torch.cuda.Stream()
    share = B.Pool(layers=len(owned), page_size=P, subs=subs, device_slots=S, host_pages=H,
                   device_layers=[[dev[b][l] for l in owned] for b in range(len(subs))], host=host, stream=stream)
    xpool = B.Pool(layers=L, page_size=P, subs=subs, device_slots=S, host_pages=0,
                   device_layers=[[dev[b][l] for l in range(L)] for b in range(len(subs))], host=None, stream=stream)
    try:
        d_t, h_t, d2_t = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (d, h, d2))
        torch.cuda.synchronize()
        share.write_back_all_layers(d_t, np.ascontiguousarray(h))  # this rank's layers only
        share.sync()
        need = xpool.layer_pack_bytes(h.size)
        staging = torch.empty(need, dtype=torch.uint8, device="cuda")
        done = [B.HipEvent() for _ in range(L)]
        for l in range(L):
            owner = l % world
            if rank == owner:
                share.load_back_layer(l // world, h_t, d2_t)
                xpool.layer_pack(l, d2_t, staging, done[l])  # the owner's layer is done once packed
                xpool.sync()
                buf = staging.cpu()
            else:
                buf = torch.empty(need, dtype=torch.uint8)
            dist.broadcast(buf, src=owner)
            if rank != owner and rank != skip:
                staging.copy_(buf)
                torch.cuda.synchronize()
                xpool.layer_unpack(l, staging, d2_t, done[l])
                xpool.sync()
        for ev in done:
            ev.synchronize()
        torch.cuda.synchronize()
        got = [[t[l].cpu().numpy() for l in range(L)] for t in dev]
        # the oracle's unsharded pool: every layer written back to one host pool, then loaded into d2
        g = O.Geometry(L, P, [tuple(s) for s in subs], H, S)
        host_full = np.zeros(O.host_pool_bytes(g), np.uint8)
        O.write_back(g, full0, host_full, d, h)
        want = [[a.copy() for a in row] for row in full0]
        for l in range(L):
            O.load_back_layer(g, l, want, host_full, h, d2)
        matches_oracle = all(np.array_equal(got[b][l], want[b][l]) for b in range(len(subs)) for l in range(L))
        digest = hashlib.sha256(b"".join(got[b][l].tobytes() for b in range(len(subs)) for l in range(L))).hexdigest()
        pages_fp = hashlib.sha256(np.ascontiguousarray(h).tobytes()).hexdigest()
        digests, fps = [None] * world, [None] * world
        dist.all_gather_object(digests, digest)
        dist.all_gather_object(fps, pages_fp)
        print(json.dumps({"rank": rank, "owned": owned, "matches_oracle": bool(matches_oracle),
                          "replicas_agree": len(set(digests)) == 1, "pages_agree": len(set(fps)) == 1}), flush=True)
    finally:
        xpool.close()
        share.close()
        host.free()
        dist.destroy_process_group()


if __name__ == "__main__":
    main()
