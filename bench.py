"""Benchmark of the KV page transfer hot path on one GPU.

A step is one write-back burst of every layer (device -> pinned host pool) and
one per-layer load-back burst of the same host pages into fresh device slots,
each layer recording its layer-done event.  The headline workload is the largest
configuration by bytes moved: the MHA pool in the K page | V page | pad shard
layout (48 layers, 8 KV heads x 128 dims bf16, 32-token pages, 262144 device
slots, 4096 host shards), bursts naming 2048 shards (~58k tokens, 11.4 GB each
way) in requests whose last page is partial, onto scattered device slots.  The
same line carries a second measured block for the 78-layer MLA + DSA indexer
pool (two host pools loaded in one burst of 1024 pages, a consumer kernel on a
second stream waiting on each layer-done event).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line: whole-step host-link throughput (GB/s, both directions'
bytes over the step time), per-direction rates, the host-link roofline of the
dominant kernel (HIP-event timing on the copy stream against the hipMemcpyAsync
peak measured here), the HBM roofline of the staged relayout kernel (as the path
runs it, staging chunks resident in the Infinity Cache, and with nothing of the
launch in that cache) and of the layer exchange kernels of a rank-sharded tier,
and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
DEFAULT_MAX_CTAS = 16        # the library's default grid cap for the zero-copy kernels
PCIE5_X16_GBS = 64.0         # MI355X host interface PCIe 5.0 x16: 128 GB/s published, 64 GB/s per direction


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mha_kv_split_shard_bf16")
    ap.add_argument("--second-workload", default="dsa_mla_indexer_78l",
                    help="a second workload measured in the same line (write-back + per-layer load-back with a "
                         "consumer per layer, host-link roofline); empty to skip")
    ap.add_argument("--write-back-mode", choices=["auto", "zerocopy", "staged"], default="zerocopy",
                    help="mode of the timed write-back (zero-copy: the highest burst rate; the staged mode, "
                         "which leaves concurrent compute alone, is measured beside it)")
    ap.add_argument("--staging-pages", type=int, default=0,
                    help="staging buffer in page images (0 = as many as the library's 256 MB chunk cap uses)")
    ap.add_argument("--max-ctas", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the second CPU oracle sample (0 = the usable cores, at most 16; 1 = skip it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-staged-probe", action="store_true")
    ap.add_argument("--no-duplex", action="store_true",
                    help="skip the write-back + load-back at-once measurement")
    ap.add_argument("--duplex-pairs", type=parse_pairs, default=DUPLEX_PAIRS,
                    help="(write-back mode):(its workgroup cap):(load-back workgroup cap), comma-separated")
    ap.add_argument("--duplex-only", action="store_true",
                    help="instead: only the write-back + load-back at-once measurement and its copy-engine peak")
    ap.add_argument("--pipeline-ctas", type=lambda t: tuple(int(x) for x in t.split(",")), default=(0, 256),
                    help="zero-copy grid caps for the layer-pipeline measurement (0 = the pool's setting)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead: write-back and per-layer load-back time against burst size (prefixes of "
                         "the workload's burst, 1 page up to all of it)")
    ap.add_argument("--beside-compute", action="store_true",
                    help="instead: only the write-back burst next to independent matmuls, zero-copy and staged "
                         "(for a kernel and memory-copy trace)")
    ap.add_argument("--gather-patterns", action="store_true",
                    help="instead: the staged gather's rate on the workload's burst with sequential, free-list, "
                         "page-aligned and random device slots")
    ap.add_argument("--gather-dram", action="store_true",
                    help="instead: only the staged gather with nothing of its launch in the Infinity Cache "
                         "(one chunk per call, each after a 1 GiB write on the copy stream)")
    ap.add_argument("--h2h", action="store_true",
                    help="instead: time host-to-host shard dump/load of the shard workload with 1..16 CPU workers")
    ap.add_argument("--compute-streams", type=int, default=5,
                    help="with --beside-compute: compute streams to try beside each write-back mode")
    ap.add_argument("--max-pinned-gib", type=float, default=64.0,
                    help="cap on the pinned host pool; a larger pool keeps the burst and shrinks the page count")
    ap.add_argument("--exchange-only", action="store_true",
                    help="only time the layer exchange kernels (pack / unpack) on the workload's device pool")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this size first (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# How each workload draws the device slots of its burst (workloads.burst_for).
SLOT_DRAWS = {
    "llama3_8b_mha_bf16": "free list, 50% runs of 1-64",
    "llama3_8b_mha_bf16_token_major": "free list, 50% runs of 1-64",
    "dsv3_mla_bf16": "free list, 50% runs of 1-64",
    "dsa_mla_indexer_78l": "whole page-aligned device pages, random",
    "mha_kv_split_shard_bf16": "random, no two list neighbours in adjacent slots; requests of 1-8 pages whose "
                               "last page holds 1..P-1 rows",
}

# The library caps a staging chunk at this many bytes of page images (MI355X's Infinity Cache).
STAGING_CHUNK_BYTES = 256 << 20


def memcpy_peak(hip, host_ptr: int, dev_ptr: int, nbytes: int, stream_ptr: int, h2d: bool, reps: int = 5) -> float:
    """Best hipMemcpyAsync rate (GB/s) pinned <-> device over `reps` copies of nbytes."""
    V = ctypes.c_void_p
    e0, e1 = V(), V()
    hip.hipEventCreate(ctypes.byref(e0))
    hip.hipEventCreate(ctypes.byref(e1))
    best = 1e30
    kind = 1 if h2d else 2  # hipMemcpyHostToDevice / DeviceToHost
    for _ in range(reps):
        hip.hipEventRecord(e0, V(stream_ptr))
        if h2d:
            rc = hip.hipMemcpyAsync(V(dev_ptr), V(host_ptr), ctypes.c_size_t(nbytes), kind, V(stream_ptr))
        else:
            rc = hip.hipMemcpyAsync(V(host_ptr), V(dev_ptr), ctypes.c_size_t(nbytes), kind, V(stream_ptr))
        assert rc == 0, f"hipMemcpyAsync failed {rc}"
        hip.hipEventRecord(e1, V(stream_ptr))
        hip.hipEventSynchronize(e1)
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        best = min(best, ms.value)
    hip.hipEventDestroy(e0)
    hip.hipEventDestroy(e1)
    return nbytes / (best * 1e-3) / 1e9


def memcpy_duplex_peak(hip, host_ptr: int, dev_ptr: int, nbytes: int, streams, reps: int = 5) -> dict:
    """hipMemcpyAsync D2H and H2D of nbytes each at the same time on two streams (host
    regions [0, nbytes) and [nbytes, 2 nbytes) of host_ptr, device likewise); best span of
    `reps`: the runtime's own rate in both directions at once."""
    V = ctypes.c_void_p
    sw, sr = streams
    ev = [V() for _ in range(3)]
    for e in ev:
        hip.hipEventCreate(ctypes.byref(e))
    best = None
    for _ in range(reps):
        hip.hipEventRecord(ev[0], V(sw))
        hip.hipStreamWaitEvent(V(sr), ev[0], 0)
        assert hip.hipMemcpyAsync(V(host_ptr), V(dev_ptr), ctypes.c_size_t(nbytes), 2, V(sw)) == 0
        assert hip.hipMemcpyAsync(V(dev_ptr + nbytes), V(host_ptr + nbytes), ctypes.c_size_t(nbytes), 1, V(sr)) == 0
        hip.hipEventRecord(ev[1], V(sw))
        hip.hipEventRecord(ev[2], V(sr))
        hip.hipEventSynchronize(ev[1])
        hip.hipEventSynchronize(ev[2])
        ms = [ctypes.c_float(), ctypes.c_float()]
        hip.hipEventElapsedTime(ctypes.byref(ms[0]), ev[0], ev[1])
        hip.hipEventElapsedTime(ctypes.byref(ms[1]), ev[0], ev[2])
        span = max(ms[0].value, ms[1].value)
        if best is None or span < best[0]:
            best = (span, ms[0].value, ms[1].value)
    for e in ev:
        hip.hipEventDestroy(e)
    span, d2h, h2d = best
    return {"aggregate_GBps": round(2 * nbytes / (span * 1e-3) / 1e9, 3),
            "d2h_GBps": round(nbytes / (d2h * 1e-3) / 1e9, 3), "h2d_GBps": round(nbytes / (h2d * 1e-3) / 1e9, 3),
            "bytes_each_way": nbytes}


# (write-back mode, write-back workgroup cap, load-back workgroup cap) of the duplex measurement.
# The caps decide how the two directions share the link: zero-copy host writes on 16 workgroups
# starve zero-copy host reads; copy-engine writes beside reads on 8 workgroups leave both near 45 GB/s.
DUPLEX_PAIRS = (("staged", 16, 8), ("staged", 16, 16), ("zerocopy", 16, 16), ("zerocopy", 2, 10))


def parse_pairs(text: str):
    """'staged:16:8,zerocopy:2:10' -> ((mode, write-back cap, load-back cap), ...)"""
    out = []
    for item in text.split(","):
        mode, w, r = item.split(":")
        if mode not in ("staged", "zerocopy"):
            raise argparse.ArgumentTypeError(f"unknown write-back mode {mode!r}")
        out.append((mode, int(w), int(r)))
    return tuple(out)


def gather_patterns(B, torch, np, W, make_pool, shape, burst, h_np, gather_bytes, reps=5, rounds=2):
    """k_gather_stage rate (read + write bytes over its launch time) on the burst's host tokens
    with four device-slot patterns: one sequential run, the workload's free-list draw, whole
    device pages, and a random permutation.  Rounds interleave the patterns."""
    P, S, n = shape.page_size, shape.device_slots, burst.n
    start = (S - n) // 2 // P * P
    pats = {"sequential": np.arange(start, start + n, dtype=np.int64),
            "free_list": burst.device_idx,
            "page_aligned": W.page_aligned_slots(6, S, P, -(-n // P))[:n],
            "random": W.permutation_slots(5, S, n)}
    if any(g == B.HC_PAGE_BLOCKS for g, _ in shape.subs):
        del pats["random"]  # page blocks move whole device pages only
    spool = make_pool(B.HC_MODE_STAGED)
    out = {k: [] for k in pats}
    for _ in range(rounds):
        for name, d in pats.items():
            d_t = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int64)).cuda()
            spool.write_back_all_layers(d_t, h_np)
            spool.sync()
            spool.kernel_time(0, reset=True)
            for _ in range(reps):
                spool.write_back_all_layers(d_t, h_np)
            spool.sync()
            ng, ms = spool.kernel_time(B.KIND_GATHER)
            out[name].append(round(2 * gather_bytes * reps / (ms * 1e-3) / 1e12, 3))
            log(f"[bench] gather {name}: {out[name][-1]} TB/s")
    spool.close()
    return {k: {"TBps": v} for k, v in out.items()}


def relabel_host_pages(h, page_size: int, host_pages: int, seed: int = 7):
    """The same rows of other host pages: each distinct page of the token list h is mapped to
    a distinct page that h does not name (seeded), rows kept.  None when too few pages are left."""
    import numpy as np
    uniq, inv = np.unique(h // page_size, return_inverse=True)
    rest = np.setdiff1d(np.arange(host_pages, dtype=np.int64), uniq)
    if rest.size < uniq.size:
        return None
    other = np.random.default_rng(seed).choice(rest, uniq.size, replace=False)
    return np.ascontiguousarray(other[inv.reshape(-1)] * page_size + h % page_size, dtype=np.int64)


def duplex_timing(B, torch, np, make_pool, shape, burst, d_t, h_np, d2_t, link_bytes, pairs, reps=5):
    """A write-back burst and a per-layer load-back burst of other rows at the same time:
    two pools over the same buffers, each on its own stream.  The load-back names the same
    rows of other host pages (a page-by-page relabelling of the burst's host tokens) into
    the fresh slots d2, so the two bursts touch disjoint device and host rows."""
    L = shape.layers
    h_other = relabel_host_pages(h_np, shape.page_size, shape.host_pages)
    if h_other is None:
        return None
    hl_t = torch.from_numpy(h_other).cuda()
    sw, sr = torch.cuda.Stream(), torch.cuda.Stream()
    e0, ew, er = B.HipEvent(timing=True), B.HipEvent(timing=True), B.HipEvent(timing=True)

    def run(wp, rp, do_w, do_r):
        torch.cuda.synchronize()
        e0.record(sw)
        e0.wait_on(sr)
        if do_w:
            wp.write_back_all_layers(d_t, h_np)
        if do_r:
            for l in range(L):
                rp.load_back_layer(l, hl_t, d2_t)
        ew.record(sw)
        er.record(sr)
        ew.synchronize()
        er.synchronize()
        return e0.elapsed_ms(ew), e0.elapsed_ms(er)

    def gbs(ms):
        return round(link_bytes / (ms * 1e-3) / 1e9, 3)

    rows = []
    for mode, wctas, rctas in pairs:
        wmode = B.HC_MODE_STAGED if mode == "staged" else B.HC_MODE_ZEROCOPY
        wp = make_pool(wmode, max_ctas=wctas, flags=0, stream_=sw)
        rp = make_pool(B.HC_MODE_ZEROCOPY, max_ctas=rctas, flags=0, stream_=sr)
        run(wp, rp, True, True)
        w_alone = float(np.median([run(wp, rp, True, False)[0] for _ in range(reps)]))
        r_alone = float(np.median([run(wp, rp, False, True)[1] for _ in range(reps)]))
        both = [run(wp, rp, True, True) for _ in range(reps)]
        wp.sync()
        rp.sync()
        wp.close()
        rp.close()
        span = float(np.median([max(b) for b in both]))
        rows.append({"write_back": f"{mode}, {wctas} workgroups" if mode == "zerocopy" else "staged",
                     "load_back_workgroups": rctas,
                     "alone_GBps": {"write_back": gbs(w_alone), "load_back": gbs(r_alone)},
                     "together_GBps": {"write_back": gbs(float(np.median([b[0] for b in both]))),
                                       "load_back": gbs(float(np.median([b[1] for b in both])))},
                     "together_span_ms": round(span, 3),
                     "aggregate_GBps": round(2 * link_bytes / (span * 1e-3) / 1e9, 3),
                     "one_after_the_other_GBps": round(2 * link_bytes / ((w_alone + r_alone) * 1e-3) / 1e9, 3)})
        log(f"[bench] duplex {rows[-1]}")
    return {"what": "write-back and per-layer load-back of disjoint rows at once, two pools on two streams",
            "rows": rows, "streams": (sw, sr)}


def hip_setup(B):
    """The HIP runtime through ctypes, with the signatures the peak measurements use."""
    hip = B._hip
    for name, argt in {"hipMemcpyAsync": [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_void_p], "hipEventCreate": [ctypes.POINTER(ctypes.c_void_p)],
                       "hipStreamWaitEvent": [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]}.items():
        getattr(hip, name).argtypes = argt
        getattr(hip, name).restype = ctypes.c_int
    return hip


def duplex_measurement(B, torch, np, hip, make_pool, shape, burst, d_t, h_np, d2_t, link_bytes, host, scratch,
                       nbytes, pairs, have_staging):
    """duplex_timing over `pairs`, plus the copy-engine duplex peak on the same two streams."""
    duplex = duplex_timing(B, torch, np, make_pool, shape, burst, d_t, h_np, d2_t, link_bytes,
                           [p for p in pairs if p[0] == "zerocopy" or have_staging])
    if duplex is None:
        return None
    sw, sr = duplex.pop("streams")
    duplex["roofline"] = dict(memcpy_duplex_peak(hip, host.ptr.value, scratch.data_ptr(), nbytes,
                                                 (sw.cuda_stream, sr.cuda_stream)),
                              source="hipMemcpyAsync D2H and H2D at once on two streams, best of 5")
    if duplex["rows"]:
        best = max(duplex["rows"], key=lambda r: r["aggregate_GBps"])
        duplex["best_frac_of_duplex_peak"] = round(best["aggregate_GBps"] / duplex["roofline"]["aggregate_GBps"], 4)
        preset = [r for r in duplex["rows"]
                  if r["write_back"] == "staged" and r["load_back_workgroups"] == B.HC_DUPLEX_LOAD_BACK_CTAS]
        if preset:
            duplex["preset"] = {"what": "Pool.duplex_partner: a staged write-back pool beside a zero-copy load-back "
                                        f"pool capped at HC_DUPLEX_LOAD_BACK_CTAS = {B.HC_DUPLEX_LOAD_BACK_CTAS} "
                                        "workgroups",
                                "aggregate_GBps": preset[0]["aggregate_GBps"],
                                "frac_of_duplex_peak": round(preset[0]["aggregate_GBps"]
                                                             / duplex["roofline"]["aggregate_GBps"], 4)}
    log(f"[bench] duplex copy-engine peak {duplex['roofline']}")
    return duplex


def kernel_source_digest(source: str = "kernels") -> str:
    """sha256 of a kernel source (hc_kernels.hip, or hc_exchange.hip for "exchange") with
    comments and whitespace removed: the counters stay attached to the kernels they
    measured, not to their comments."""
    import hashlib
    import re
    fname = "hc_kernels.hip" if source == "kernels" else "hc_exchange.hip"
    src = open(os.path.join(ROOT, "host_device_page_amd", "csrc", fname)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()


def counter_traffic(workload: str, kernel: str, source: str = "kernels"):
    """Bytes per launch that the FETCH_SIZE / WRITE_SIZE counter passes measured for
    `kernel` (scaled by the known-size copy), from the committed profile summary, or
    None when the kernel source changed since the counters were taken.  source:
    "kernels" (the transfer kernels) or "exchange" (the layer exchange kernels)."""
    suffix = "_counters.json" if source == "kernels" else "_exchange_counters.json"
    path = os.path.join(ROOT, "profiles", f"{workload}{suffix}")
    if not os.path.exists(path):
        return None
    prof = json.load(open(path))
    if prof.get("kernel_code_digest") != kernel_source_digest(source):
        return None
    k = prof["kernels"].get(kernel)
    if not k:
        return None
    return {"bytes": int(k["fetch_bytes"] + k["write_bytes"]), "fetch_bytes": int(k["fetch_bytes"]),
            "write_bytes": int(k["write_bytes"]), "source": os.path.relpath(path, ROOT)}


def burst_bytes(shape, burst) -> tuple[int, int]:
    """Algorithmic bytes of one burst: every named token row of every layer, plus page
    blocks once per page; (host-link bytes, shard pad bytes written)."""
    P, L = shape.page_size, shape.layers
    rows = sum(e for g, e in shape.subs if g == 0)
    blocks = sum(e for g, e in shape.subs if g == 1)
    n = burst.n
    whole_pages = int((burst.host_idx % P == 0).sum())
    return L * (n * rows + whole_pages * blocks), 0


def staged_bytes(shape, burst) -> int:
    """Bytes one burst moves through the staged gather: the rows (and page blocks) of every
    wholly named host page, over all layers.  Rows of pages the burst names in part go
    through the zero-copy kernel instead (rows it does not name must stay as they are),
    so they are not the gather's."""
    import numpy as np
    P, L = shape.page_size, shape.layers
    _, counts = np.unique(burst.host_idx // P, return_counts=True)
    whole = int((counts == P).sum())
    rows = sum(e for g, e in shape.subs if g == 0)
    blocks = sum(e for g, e in shape.subs if g == 1)
    return L * whole * (P * rows + blocks)


def gather_dram_bound(B, torch, np, W, make_pool, stream, shape, burst, chunk_pages, reps=5):
    """k_gather_stage with nothing of its launch in MI355X's 256 MB Infinity Cache.  Each
    write-back call names exactly one staging chunk of wholly named pages (the burst's
    first ones), and each follows a 1 GiB write on the copy stream, which leaves the cache
    full of other dirty lines: the gather reads its rows from DRAM, and its staging writes
    displace dirty lines that go to DRAM.  The same chunk without the write, back to back,
    is timed beside it.  Bytes per launch: the chunk's rows read plus the same written."""
    P = shape.page_size
    pg = burst.host_idx // P
    uniq, counts = np.unique(pg, return_counts=True)
    whole = set(uniq[counts == P].tolist())
    pick = [int(p) for p in burst.pages if int(p) in whole][:chunk_pages]
    mask = np.isin(pg, pick)
    d = np.ascontiguousarray(burst.device_idx[mask])
    h = np.ascontiguousarray(burst.host_idx[mask])
    nbytes = staged_bytes(shape, W.Burst(d, h, np.array(pick, dtype=np.int64)))
    d_t = torch.from_numpy(d).cuda()
    spool = make_pool(B.HC_MODE_STAGED)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    spool.write_back_all_layers(d_t, h)
    spool.sync()
    res = {}
    # the runtime's plain device-to-device copy of the same bytes under the same condition
    # (after the same 1 GiB write), for reference
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    cms = []
    for k in range(reps):
        with torch.cuda.stream(stream):
            flush.fill_(k & 0xFF)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
        e1.synchronize()
        cms.append(e0.elapsed_ms(e1))
    res["plain_copy_same_condition_GBps"] = round(2 * nbytes / (float(np.median(cms)) * 1e-3) / 1e9, 1)
    del src, dst
    for name, flushed in (("dram", True), ("back_to_back", False)):
        spool.kernel_time(0, reset=True)
        for k in range(reps):
            if flushed:
                with torch.cuda.stream(stream):
                    flush.fill_(k & 0xFF)
            spool.write_back_all_layers(d_t, h)
        spool.sync()
        n_g, ms_g = spool.kernel_time(B.KIND_GATHER)
        assert n_g == reps, f"expected one gather launch per call, got {n_g} for {reps}"
        res[name] = {"avg_launch_ms": round(ms_g / n_g, 4),
                     "achieved": round(2 * nbytes / (ms_g / n_g * 1e-3) / 1e9, 1)}
    spool.close()
    del flush
    return {"chunk_pages": len(pick), "bytes_per_launch": 2 * nbytes, "flush_bytes": 1 << 30, **res}


def plain_copy_dram(B, torch, np, stream, nbytes: int = 2 << 30, reps: int = 5) -> float:
    """The runtime's plain device-to-device copy (torch copy_) of 2 GiB, 8 times the Infinity
    Cache, so both sides stream from and to DRAM: a reference for what this memory system
    copies (read + write bytes over the copy's time, best of `reps`)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    best = None
    for _ in range(reps):
        with torch.cuda.stream(stream):
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_ms(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return round(2 * nbytes / (best * 1e-3) / 1e9, 1)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _page_cuts(h, page_size: int, parts: int):
    """Cut positions of the index list into about `parts` slices, each cut at a
    change of host page, so no host page (nor its shard pad) is shared."""
    import numpy as np
    pg = h // page_size
    starts = np.flatnonzero(np.r_[True, pg[1:] != pg[:-1]])
    cuts = sorted({int(starts[np.searchsorted(starts, k * h.size // parts)]) if k * h.size // parts <= starts[-1]
                   else h.size for k in range(1, parts)})
    return [0] + [c for c in cuts if 0 < c < h.size] + [h.size]


def cpu_baseline(shape, burst, d2, seconds: float, threads: int = 1):
    """The oracle, as written, on host-memory replicas: write-back then load-back of
    the full burst restricted to layer 0 of the pool (1 of L layers), repeated
    until `seconds` pass.  With threads > 1 the burst is cut at host-page changes
    into one slice per thread; every thread calls the same oracle functions on its
    slice (disjoint rows, pages and slots, so together they do the whole burst),
    like a pool of CPU copy workers.  The rate counts the bytes of every finished
    slice pass over the time until the last thread stops."""
    import threading

    import numpy as np

    from oracle import oracle as O
    g1 = O.Geometry(1, shape.page_size, list(shape.subs), shape.host_pages, shape.device_slots,
                    shape.layout, shape.align)
    dev = [[np.ones(g1.device_units(b) * e, dtype=np.uint8)] for b, (_, e) in enumerate(shape.subs)]
    host = np.ones(O.host_pool_bytes(g1), dtype=np.uint8)

    def pass_bytes(h):  # write-back + load-back bytes of one pass over these tokens
        return 2 * sum(h.size * e if g == 0 else int((h % shape.page_size == 0).sum()) * e for g, e in shape.subs)

    cuts = _page_cuts(burst.host_idx, shape.page_size, threads)
    slices = [(burst.device_idx[a:b], burst.host_idx[a:b], d2[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    done = [0] * len(slices)
    t0 = time.perf_counter()
    deadline = t0 + seconds

    def work(k):
        d, h, f = slices[k]
        while True:
            O.write_back(g1, dev, host, d, h)
            O.load_back_layer(g1, 0, dev, host, h, f)
            done[k] += 1
            if time.perf_counter() >= deadline:
                return

    if len(slices) == 1:
        work(0)
    else:
        ts = [threading.Thread(target=work, args=(k,)) for k in range(len(slices))]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    el = time.perf_counter() - t0
    moved = sum(done[k] * pass_bytes(slices[k][1]) for k in range(len(slices)))
    how = "single thread" if len(slices) == 1 else f"{len(slices)} threads on disjoint page-aligned slices"
    return {"value": round(moved / el / 1e9, 3), "unit": "GB/s", "cores": len(slices), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"C oracle write-back + load-back of the full {burst.n}-token burst on layer 0 only "
                      f"(1 of {shape.layers} layers, same rows/pages/index lists), {sum(done)} slice passes in "
                      f"{el:.1f} s, {how}, host-RAM replicas of the device pool and the host pool"}


def cpu_exchange_baseline(shape, burst, d2, seconds: float):
    """The oracle's layer exchange, as written, on a host-memory replica of layer 0: pack
    the burst's slots, unpack them into a second replica, repeated until `seconds` pass,
    on one thread.  Counted like the GPU kernels: each of the two calls reads and writes
    the layer's packed bytes."""
    import numpy as np

    from oracle import oracle as O
    g1 = O.Geometry(1, shape.page_size, list(shape.subs), 1, shape.device_slots, shape.layout, shape.align)
    owner = [[np.ones(g1.device_units(b) * e, dtype=np.uint8)] for b, (_, e) in enumerate(shape.subs)]
    other = [[np.full(g1.device_units(b) * e, 2, dtype=np.uint8)] for b, (_, e) in enumerate(shape.subs)]
    packed_bytes = O.layer_packed_bytes(g1, d2.size)
    O.layer_unpack(g1, 0, other, d2, O.layer_pack(g1, 0, owner, d2))  # untimed: first touch of the pages
    passes = 0
    t0 = time.perf_counter()
    while True:
        O.layer_unpack(g1, 0, other, d2, O.layer_pack(g1, 0, owner, d2))
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(4 * packed_bytes * passes / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"C oracle pack + unpack of layer 0 at the burst's {d2.size} load-back slots "
                      f"({packed_bytes} packed bytes), {passes} passes in {el:.1f} s, single thread, host-RAM replicas"}


def layer_pipeline(B, torch, pool, shape, h_t, d2_t, n, stream, layer_events, make_pool, args):
    """Overlap of the per-layer load-back with a consumer on a second stream.  The
    consumer's work per layer is a bf16 matmul sized to about one layer's transfer
    time; it waits on the layer's event before it starts.  overlap = (load + consume
    - both) / min(load, consume): 1 when the shorter one hides completely."""
    import numpy as np
    L = shape.layers
    consumer = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    out = torch.empty(4096, 4096, device="cuda", dtype=torch.bfloat16)
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def one_matmul():
        with torch.cuda.stream(consumer):
            torch.matmul(a, w, out=out)
    for _ in range(3):
        timed(one_matmul)
    per_mm = float(np.median([timed(one_matmul) for _ in range(5)]))
    res = {"consumer": "bf16 matmul 4096^3 x k per layer, on a second stream, after hipStreamWaitEvent(layer event)"}
    for ctas in args.pipeline_ctas:
        p = pool if ctas == 0 else make_pool(B.HC_MODE_ZEROCOPY, max_ctas=ctas)

        def load():
            for l in range(L):
                p.load_back_layer(l, h_t, d2_t, layer_events[l])
        t_load = float(np.median([timed(load) for _ in range(3)]))
        reps = max(1, int(round(t_load / L / max(per_mm, 1e-6))))

        def consume_only():
            with torch.cuda.stream(consumer):
                for _ in range(L * reps):
                    torch.matmul(a, w, out=out)

        def both():
            for l in range(L):
                p.load_back_layer(l, h_t, d2_t, layer_events[l])
                layer_events[l].wait_on(consumer)
                with torch.cuda.stream(consumer):
                    for _ in range(reps):
                        torch.matmul(a, w, out=out)
        t_cons = float(np.median([timed(consume_only) for _ in range(3)]))
        t_both = float(np.median([timed(both) for _ in range(3)]))
        ov = (t_load + t_cons - t_both) / min(t_load, t_cons)
        key = f"max_ctas_{ctas or args.max_ctas or DEFAULT_MAX_CTAS}"
        res[key] = {"load_ms": round(t_load * 1e3, 3), "consume_ms": round(t_cons * 1e3, 3),
                    "both_ms": round(t_both * 1e3, 3), "matmuls_per_layer": reps, "overlap": round(ov, 4),
                    "load_GBps_alone": round(n * L * sum(e for _, e in shape.subs) / t_load / 1e9, 2)}
        log(f"[bench] layer pipeline {key}: {res[key]}")
        if p is not pool:
            p.close()
    return res


def write_back_overlap(B, torch, np, pools, d_t, h_np, consumers: int = 3):
    """A whole write-back burst next to independent compute (bf16 4096^3 matmuls on another
    stream, about as long as the burst), per write-back mode, once for each of `consumers`
    compute streams: HIP maps a process's streams onto GPU_MAX_HW_QUEUES hardware queues, so
    whether a compute stream shares a queue with a stream of the write-back (and then waits
    behind it) depends on the stream.  overlap = (write-back + compute - both) /
    min(write-back, compute) per compute stream; `overlap` is their median."""
    streams = [torch.cuda.Stream() for _ in range(consumers)]
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    out = torch.empty(4096, 4096, device="cuda", dtype=torch.bfloat16)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def matmuls(cs, k):
        with torch.cuda.stream(cs):
            for _ in range(k):
                torch.matmul(a, w, out=out)
    for _ in range(3):
        timed(lambda: matmuls(streams[0], 1))
    per_mm = float(np.median([timed(lambda: matmuls(streams[0], 1)) for _ in range(5)]))
    res = {"compute": "bf16 matmul 4096^3 repeated on another stream, no dependency on the burst",
           "compute_streams": consumers,
           "hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "4 (HIP default)")}
    for mode, p in pools.items():
        p.write_back_all_layers(d_t, h_np)
        t_wb = float(np.median([timed(lambda: p.write_back_all_layers(d_t, h_np)) for _ in range(3)]))
        k = max(1, int(round(t_wb / max(per_mm, 1e-6))))
        rows = []
        for cs in streams:
            t_c = float(np.median([timed(lambda: matmuls(cs, k)) for _ in range(3)]))

            def both():
                p.write_back_all_layers(d_t, h_np)
                matmuls(cs, k)
            t_both = float(np.median([timed(both) for _ in range(3)]))
            rows.append({"compute_ms": round(1e3 * t_c, 3), "both_ms": round(1e3 * t_both, 3),
                         "overlap": round((t_wb + t_c - t_both) / min(t_wb, t_c), 4)})
        ovs = [r["overlap"] for r in rows]
        res[mode] = {"write_back_ms": round(1e3 * t_wb, 3), "matmuls": k, "overlap": float(np.median(ovs)),
                     "overlap_by_compute_stream": ovs, "compute_ms": rows[0]["compute_ms"],
                     "both_ms": [r["both_ms"] for r in rows]}
        log(f"[bench] write-back beside compute, {mode}: {res[mode]}")
    return res


def h2h_main(args):
    """Host-to-host shard dump + load of 512 pages of the 48-layer K|V shard workload
    (3 MiB + 3 MiB per shard) between two host buffers, for several worker counts."""
    import numpy as np

    from host_device_page_amd import binding as B
    from host_device_page_amd import workloads as W
    shape = W.SHAPES["mha_kv_split_shard_bf16"]
    L, P = shape.layers, shape.page_size
    n = 512
    subs = [(g, e, [16] * L) for g, e in shape.subs]
    d_pf, _k1 = B.make_desc(layers=L, page_size=P, subs=subs, device_slots=shape.device_slots, host_pages=n,
                            layout=B.HC_LAYOUT_PAGE_FIRST)
    d_sh, _k2 = B.make_desc(layers=L, page_size=P, subs=subs, device_slots=shape.device_slots, host_pages=n,
                            layout=B.HC_LAYOUT_KV_SPLIT_SHARD, shard_align=shape.align)
    host = np.ones(B.host_pool_bytes(d_pf), dtype=np.uint8)
    store = np.ones(B.host_pool_bytes(d_sh), dtype=np.uint8)
    stride = B.staging_page_bytes(d_sh)
    sizes = [L * P * e for _, e in shape.subs]
    order = np.random.default_rng(1).permutation(n)
    pages = [[host.ctypes.data + B.host_offset(d_pf, b, int(p), 0, 0) for b in range(len(sizes))] for p in order]
    shards = [store.ctypes.data + q * stride for q in range(n)]
    payload = n * sum(sizes)
    out = {"metric": "host-to-host shard copy GB/s", "unit": "GB/s", "shards": n, "shard_bytes": stride,
           "payload_bytes": payload, "cpu_threads_available": len(os.sched_getaffinity(0)), "by_workers": {}}
    for w in (1, 2, 4, 8, 16):
        eng = B.H2H(workers=w, queue_depth=4096)
        eng.wait(eng.submit(B.HC_H2H_DUMP, sizes, pages, shards, stride))  # warm
        res = {}
        for name, direction in (("dump", B.HC_H2H_DUMP), ("load", B.HC_H2H_LOAD)):
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                eng.wait(eng.submit(direction, sizes, pages, shards, stride))
                ts.append(time.perf_counter() - t0)
            res[name] = round(payload / float(np.median(ts)) / 1e9, 2)
        eng.close()
        out["by_workers"][w] = res
        log(f"[h2h] workers {w}: {res}")
    print(json.dumps(out), flush=True)


def calibration_copy(torch, mib: int) -> None:
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    if not mib:
        return
    nb = mib << 20
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {nb} bytes done")
    del src, dst


def layer_exchange_timing(B, np, shape, dev, d_t, n, stream, counter_workload=None, rounds=2):
    """The per-layer exchange of a rank-sharded host tier (the owner packs a loaded layer's
    rows into staging, the other ranks unpack them), on a device-only pool over the
    workload's device buffers: every layer packed into its own staging buffer, then every
    layer unpacked from it, `rounds` times, with per-launch HIP-event timing.  Each launch
    finds its rows and its staging cold (the layers cycle through more than the 256 MB
    Infinity Cache), as a receiving rank's unpack after the broadcast would.  Unpack puts
    back the bytes pack took, so the pool is unchanged.  Algorithmic bytes per launch: the
    layer's packed bytes read plus the same written.  For scale, a plain device-to-device
    copy of the same bytes is timed too."""
    import torch
    L = shape.layers
    xpool = B.Pool(layers=L, page_size=shape.page_size, subs=list(shape.subs), device_slots=shape.device_slots,
                   host_pages=0, device_layers=[[t[l] for l in range(L)] for t in dev], host=None, stream=stream,
                   flags=B.HC_FLAG_PROFILE)
    packed = xpool.layer_pack_bytes(n)
    staging = torch.empty((L, packed), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    xpool.layer_pack(0, d_t, staging[0])
    xpool.layer_unpack(0, staging[0], d_t)
    xpool.sync()
    xpool.kernel_time(B.KIND_PACK, reset=True)
    for _ in range(rounds):
        for l in range(L):
            xpool.layer_pack(l, d_t, staging[l])
        for l in range(L):
            xpool.layer_unpack(l, staging[l], d_t)
    n_p, ms_p = xpool.kernel_time(B.KIND_PACK)
    n_u, ms_u = xpool.kernel_time(B.KIND_UNPACK)
    # As the path runs it: the owner's pack is read right away (by the broadcast; here by the
    # unpack), so each layer is packed into one staging buffer and unpacked from it at once.
    xpool.kernel_time(B.KIND_PACK, reset=True)
    for _ in range(rounds):
        for l in range(L):
            xpool.layer_pack(l, d_t, staging[0])
            xpool.layer_unpack(l, staging[0], d_t)
    n_wp, ms_wp = xpool.kernel_time(B.KIND_PACK)
    n_wu, ms_wu = xpool.kernel_time(B.KIND_UNPACK)
    xpool.sync()
    xpool.close()
    # the same bytes through a plain copy, source and destination as cold as the kernels'
    # (rows half the layer count apart, so neither was touched recently)
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    half = max(1, L // 2)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(rounds):
            for l in range(L):
                staging[(l + half) % L].copy_(staging[l])
        e1.record(stream)
    e1.synchronize()
    copies = rounds * L if L > 1 else 0
    copy_gbs = 2 * packed * copies / (e0.elapsed_ms(e1) * 1e-3) / 1e9 if copies else None
    del staging
    out = {"layer_packed_bytes": packed, "tokens": n, "launches": {"pack": n_p, "unpack": n_u},
           "plain_copy_same_bytes_GBps": round(copy_gbs, 1) if copy_gbs else None}
    for name, cnt, ms, kname in (("pack", n_p, ms_p, "k_layer_exchange<true>"),
                                 ("unpack", n_u, ms_u, "k_layer_exchange<false>")):
        avg = ms / max(1, cnt)
        gbs = 2 * packed / (avg * 1e-3) / 1e9
        traffic = counter_traffic(counter_workload, kname, "exchange") if counter_workload else None
        out[name] = {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(avg, 5),
                     "bytes_per_launch": 2 * packed, "traffic": traffic["bytes"] if traffic else None}
    out["cold"] = "each layer packed into its own staging buffer, then each unpacked (rows and staging cold)"
    pair_ms = ms_wp / max(1, n_wp) + ms_wu / max(1, n_wu)
    out["warm_pair"] = {
        "what": "pack then unpack of each layer on one staging buffer, back to back (the packed layer is read "
                "right after it is written)",
        "pack_avg_launch_ms": round(ms_wp / max(1, n_wp), 5), "unpack_avg_launch_ms": round(ms_wu / max(1, n_wu), 5),
        "pack_GBps": round(2 * packed / (ms_wp / max(1, n_wp) * 1e-3) / 1e9, 1),
        "unpack_GBps": round(2 * packed / (ms_wu / max(1, n_wu) * 1e-3) / 1e9, 1),
        "pair_GBps": round(4 * packed / (pair_ms * 1e-3) / 1e9, 1),
        "pair_frac": round(4 * packed / (pair_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def load_back_graph_timing(B, np, pool, stream, L, h, d, link_bytes, reps=7):
    """The per-layer load-back of (h, d) as one captured graph against the same L calls
    made eagerly, on an unprofiled pool: GPU time per layer (HIP events on the copy
    stream) and CPU time to enqueue the burst, medians after 2 warm-up repetitions."""
    events = [B.HipEvent() for _ in range(L)]
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    graph = pool.capture_load_back(h, d, events)
    g_ms, g_cpu, e_ms, e_cpu = [], [], [], []
    for _ in range(reps):
        e0.record(stream)
        t0 = time.perf_counter()
        graph.launch()
        g_cpu.append(time.perf_counter() - t0)
        e1.record(stream)
        e1.synchronize()
        g_ms.append(e0.elapsed_ms(e1))
        e0.record(stream)
        t0 = time.perf_counter()
        for l in range(L):
            pool.load_back_layer(l, h, d, events[l])
        e_cpu.append(time.perf_counter() - t0)
        e1.record(stream)
        e1.synchronize()
        e_ms.append(e0.elapsed_ms(e1))
    graph.close()
    med = lambda v: float(np.median(v[2:]))
    return {"graph_ms_per_layer": round(med(g_ms) / L, 4), "eager_ms_per_layer": round(med(e_ms) / L, 4),
            "graph_GBps": round(link_bytes / (med(g_ms) * 1e6), 3), "eager_GBps": round(link_bytes / (med(e_ms) * 1e6), 3),
            "graph_cpu_ms_per_burst": round(1e3 * med(g_cpu), 4), "eager_cpu_ms_per_burst": round(1e3 * med(e_cpu), 4)}


def burst_size_sweep(B, np, pool, shape, stream, burst, d_t, h_np, h_t, d2_t, args):
    """Latency and rate against burst size: the first k pages' tokens of the
    workload's burst, k = 1, 2, 4, ... up to the whole burst.  Write-back: one call
    bracketed by HIP events on the copy stream, plus its CPU enqueue time.
    Load-back: one layer alone, and all layers back to back (per-layer average)."""
    P, L = shape.page_size, shape.layers
    pg = burst.host_idx // P
    starts = np.flatnonzero(np.r_[True, pg[1:] != pg[:-1]])
    ends = np.r_[starts[1:], burst.n]
    ks = []
    k = 1
    while k < starts.size:
        ks.append(k)
        k *= 2
    ks.append(int(starts.size))
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    layer_events = [B.HipEvent() for _ in range(L)]
    rows = []
    for k in ks:
        n = int(ends[k - 1])
        sub = type(burst)(burst.device_idx[:n], burst.host_idx[:n], burst.pages[:k])
        link, _ = burst_bytes(shape, sub)
        d, h, hd, d2 = d_t[:n], h_np[:n], h_t[:n], d2_t[:n]
        wb, cpu, one, chain = [], [], [], []
        for rep in range(7):
            e0.record(stream)
            t0 = time.perf_counter()
            pool.write_back_all_layers(d, h)
            cpu.append(time.perf_counter() - t0)
            e1.record(stream)
            e1.synchronize()
            wb.append(e0.elapsed_ms(e1))
            e0.record(stream)
            pool.load_back_layer(0, hd, d2, layer_events[0])
            e1.record(stream)
            e1.synchronize()
            one.append(e0.elapsed_ms(e1))
            e0.record(stream)
            for l in range(L):
                pool.load_back_layer(l, hd, d2, layer_events[l])
            e1.record(stream)
            e1.synchronize()
            chain.append(e0.elapsed_ms(e1))
        # the first two repetitions warm up
        g = load_back_graph_timing(B, np, pool, stream, L, hd, d2, link)
        wb_ms, cpu_ms = float(np.median(wb[2:])), 1e3 * float(np.median(cpu[2:]))
        one_ms, chain_ms = float(np.median(one[2:])), float(np.median(chain[2:])) / L
        rows.append({"pages": k, "tokens": n, "bytes_each_way": link,
                     "write_back_ms": round(wb_ms, 4), "write_back_GBps": round(link / (wb_ms * 1e6), 2),
                     "write_back_cpu_ms": round(cpu_ms, 4),
                     "load_back_one_layer_ms": round(one_ms, 4),
                     "load_back_ms_per_layer_chained": round(chain_ms, 4),
                     "load_back_GBps_chained": round(link / L / (chain_ms * 1e6), 2),
                     "load_back_ms_per_layer_graph": g["graph_ms_per_layer"],
                     "load_back_graph_cpu_ms": g["graph_cpu_ms_per_burst"],
                     "load_back_eager_cpu_ms": g["eager_cpu_ms_per_burst"]})
        log(f"[sweep] {rows[-1]}")
    pool.sync()
    return rows


def staged_probe(B, torch, np, W, make_pool, stream, shape, burst, d_t, h_np, link_bytes, reps, chunk_pages):
    """The same burst through the staged write-back: the HBM roofline of k_gather_stage as the
    path runs it (chunks of page images capped to stay in the Infinity Cache until the copy
    engines read them), the same kernel with nothing of its launch in that cache, and the
    staged burst's rate."""
    spool = make_pool(B.HC_MODE_STAGED)
    for _ in range(2):
        spool.write_back_all_layers(d_t, h_np)
    spool.sync()
    spool.kernel_time(0, reset=True)
    e0, e1 = B.HipEvent(timing=True), B.HipEvent(timing=True)
    sms = []
    for _ in range(reps):
        e0.record(stream)
        spool.write_back_all_layers(d_t, h_np)
        e1.record(stream)
        e1.synchronize()
        sms.append(e0.elapsed_ms(e1))
    n_g, ms_g = spool.kernel_time(B.KIND_GATHER)
    n_c, ms_c = spool.kernel_time(B.KIND_COPY_ENGINE)
    spool.sync()
    spool.close()
    gbytes = staged_bytes(shape, burst)           # what the gather moves: wholly named pages
    chunks = n_g // reps
    g_gbs = 2 * gbytes * reps / (ms_g * 1e-3) / 1e9  # read + write of every gathered byte
    gtraffic = counter_traffic(shape.name, "k_gather_stage")
    dram = gather_dram_bound(B, torch, np, W, make_pool, stream, shape, burst, chunk_pages)
    copy_ref = plain_copy_dram(B, torch, np, stream)
    d_gbs = dram["dram"]["achieved"]
    dtraffic = counter_traffic(shape.name, "k_gather_stage_dram")
    roofline_hbm = {"bound": "hbm", "kernel": "k_gather_stage (staged lf->pf relayout, one chunk, all layers)",
                    "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                    "traffic": gtraffic["bytes"] if gtraffic else None,
                    "avg_launch_ms": round(ms_g / n_g, 4), "bytes_per_launch": int(2 * gbytes / max(1, chunks)),
                    "chunk_pages": chunk_pages, "gathered_bytes_per_burst": gbytes,
                    "staging": "as the path runs: chunks capped at 256 MB so the copy engines read the page images "
                               "the gather just wrote from the Infinity Cache; part of the write side stays in that "
                               "cache, so this rate is an upper bound for DRAM alone",
                    "dram_bound": {"achieved": d_gbs, "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                                   "avg_launch_ms": dram["dram"]["avg_launch_ms"],
                                   "bytes_per_launch": dram["bytes_per_launch"], "chunk_pages": dram["chunk_pages"],
                                   "back_to_back_achieved": dram["back_to_back"]["achieved"],
                                   "plain_copy_same_condition_GBps": dram["plain_copy_same_condition_GBps"],
                                   "traffic": dtraffic["bytes"] if dtraffic else None,
                                   "method": "one chunk of wholly named pages per call, each call after a 1 GiB "
                                             "write on the copy stream (rows read from DRAM, staging writes "
                                             "displace dirty lines)"},
                    "plain_copy_dram_GBps": copy_ref,
                    "meets_70pct_of_peak": {"as_run": g_gbs >= 0.7 * HBM_PEAK_GBS,
                                            "dram_bound": d_gbs >= 0.7 * HBM_PEAK_GBS}}
    staged = {"write_back_GBps": round(link_bytes / (float(np.median(sms)) * 1e-3) / 1e9, 3),
              "copy_engine_ms_per_burst": round(ms_c / reps, 3),
              "gather_ms_per_burst": round(ms_g / reps, 3)}
    log(f"[bench] gather {g_gbs:.1f} GB/s as run, {d_gbs} GB/s with nothing in the Infinity Cache")
    return roofline_hbm, staged


def second_block(args, name: str, peaks: dict) -> dict:
    """A second workload in the same line: K timed steps of write-back (zero-copy) + per-layer
    load-back, where a consumer stream waits on each layer-done event and runs a small kernel
    that reads the loaded layer (the dummy attention of the 78-layer two-pool burst); the
    host-link roofline of its dominant kernel against the peaks measured for the headline; and
    the staged gather's HBM rates."""
    import numpy as np
    import torch

    from host_device_page_amd import binding as B
    from host_device_page_amd import workloads as W
    shape = capped_shape(B, W, name, args.max_pinned_gib)
    L, P = shape.layers, shape.page_size
    log(f"[bench] second workload {shape.name}: L={L} P={P} subs={shape.subs} S={shape.device_slots} "
        f"H={shape.host_pages}")
    t_setup = time.perf_counter()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    dev = []
    for g, e in shape.subs:
        units = shape.device_slots // P if g == 1 else shape.device_slots
        dev.append(torch.empty((L, units * e), dtype=torch.uint8, device="cuda").random_(0, 256, generator=gen))
    probe, _k = B.make_desc(layers=L, page_size=P, subs=[(g, e, [1] * L) for g, e in shape.subs],
                            device_slots=shape.device_slots, host_pages=shape.host_pages, layout=shape.layout,
                            shard_align=shape.align)
    host = B.HostBuffer(B.host_pool_bytes(probe))
    img = B.staging_page_bytes(probe)
    chunk_pages = max(1, STAGING_CHUNK_BYTES // img)
    staging = torch.empty(chunk_pages * img, dtype=torch.uint8, device="cuda")
    stream, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    layers = [[t[l] for l in range(L)] for t in dev]

    def make_pool(mode, max_ctas=None, flags=B.HC_FLAG_PROFILE, stream_=None):
        return B.Pool(layers=L, page_size=P, subs=list(shape.subs), device_slots=shape.device_slots,
                      host_pages=shape.host_pages, device_layers=layers, host=host,
                      stream=stream if stream_ is None else stream_, layout=shape.layout, shard_align=shape.align,
                      staging=staging, write_back_mode=mode, flags=flags,
                      max_ctas=args.max_ctas if max_ctas is None else max_ctas)

    pool = make_pool(B.HC_MODE_ZEROCOPY)
    burst = W.burst_for(shape, seed=1)
    d2 = W.fresh_slots_like(shape, burst, seed=2)
    d_t = torch.from_numpy(burst.device_idx).cuda()
    h_np = np.ascontiguousarray(burst.host_idx)
    h_t = torch.from_numpy(h_np).cuda()
    d2_t = torch.from_numpy(d2).cuda()
    link_bytes, _ = burst_bytes(shape, burst)
    seen = torch.zeros((L, 16), dtype=torch.uint8, device="cuda")
    layer_events = [B.HipEvent() for _ in range(L)]
    ev_wb0, ev_wb1, ev_lb1, ev_c = (B.HipEvent(timing=True) for _ in range(4))
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; burst {burst.n} tokens, {burst.pages.size} pages")

    def step():
        ev_wb0.record(stream)
        pool.write_back_all_layers(d_t, h_np)
        ev_wb1.record(stream)
        for l in range(L):
            pool.load_back_layer(l, h_t, d2_t, layer_events[l])
            layer_events[l].wait_on(consumer)
            with torch.cuda.stream(consumer):
                seen[l].copy_(dev[0][l][:16])  # reads the layer once its event has completed
        ev_lb1.record(stream)
        ev_c.record(consumer)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pool.kernel_time(0, reset=True)
    wb_ms, lb_ms, c_ms = [], [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
        ev_c.synchronize()
        ev_lb1.synchronize()
        wb_ms.append(ev_wb0.elapsed_ms(ev_wb1))
        lb_ms.append(ev_wb1.elapsed_ms(ev_lb1))
        c_ms.append(ev_wb1.elapsed_ms(ev_c))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    n_rd, ms_rd = pool.kernel_time(B.KIND_ZC_READ)
    n_wr, ms_wr = pool.kernel_time(B.KIND_ZC_WRITE)
    pool.sync()
    pool.close()
    wb_gbs = link_bytes / (float(np.median(wb_ms)) * 1e-3) / 1e9
    lb_gbs = link_bytes / (float(np.median(lb_ms)) * 1e-3) / 1e9
    per_layer = link_bytes // L
    if n_wr and ms_wr > ms_rd:
        kname, avg, nbytes, peak = "k_zc_write", ms_wr / n_wr, link_bytes, peaks["d2h"]
    else:
        kname, avg, nbytes, peak = "k_zc_read", ms_rd / max(1, n_rd), per_layer, peaks["h2d"]
    achieved = nbytes / (avg * 1e-3) / 1e9
    traffic = counter_traffic(shape.name, kname)
    roofline = {"bound": "host_link", "kernel": kname, "achieved": round(achieved, 3), "peak": round(peak, 3),
                "unit": "GB/s", "frac": round(achieved / peak, 4), "traffic": traffic["bytes"] if traffic else None,
                "avg_launch_ms": round(avg, 4), "bytes_per_launch": nbytes,
                "launches": n_rd if kname == "k_zc_read" else n_wr,
                "peak_source": "hipMemcpyAsync pinned<->device 1 GiB best of 5, measured for the headline workload",
                "frac_of_published": round(achieved / PCIE5_X16_GBS, 4)}
    roofline_hbm, staged = staged_probe(B, torch, np, W, make_pool, stream, shape, burst, d_t, h_np, link_bytes,
                                        max(3, args.steps // 2), chunk_pages)
    host.free()
    del dev, staging, layers
    return {"workload": shape.name, "layers": L, "page_size": P, "row_bytes": list(shape.row_bytes),
            "device_slots": shape.device_slots, "host_pages": shape.host_pages,
            "burst_pages": int(burst.pages.size), "burst_tokens": burst.n, "burst_bytes_each_way": link_bytes,
            "steps": args.steps, "warmup": args.warmup,
            "value": round(2 * link_bytes * args.steps / el / 1e9, 3), "unit": "GB/s",
            "ms_per_step": round(el * 1e3 / args.steps, 3),
            "write_back_GBps": round(wb_gbs, 3), "load_back_GBps": round(lb_gbs, 3),
            "frac_of_link_peak": {"write_back": round(wb_gbs / peaks["d2h"], 4),
                                  "load_back": round(lb_gbs / peaks["h2d"], 4)},
            "load_back_with_consumer": {
                "consumer": "after hipStreamWaitEvent(layer event) on a second stream, a 16-byte copy out of the "
                            "loaded layer, per layer",
                "consumer_done_after_load_back_ms": round(float(np.median(c_ms)) - float(np.median(lb_ms)), 4),
                "GBps_to_last_consumer": round(link_bytes / (float(np.median(c_ms)) * 1e-3) / 1e9, 3)},
            "pages_per_s": round(2 * burst.pages.size * args.steps / el, 1),
            "roofline": roofline, "roofline_hbm": roofline_hbm, "staged_write_back": staged}


def capped_shape(B, W, name: str, max_pinned_gib: float):
    """The workload's pool shape with as many host pages as the pinned-memory cap holds."""
    shape = W.SHAPES[name]
    L, P = shape.layers, shape.page_size
    one, _k1 = B.make_desc(layers=L, page_size=P, subs=[(g, e, [1] * L) for g, e in shape.subs],
                           device_slots=shape.device_slots, host_pages=1, layout=shape.layout, shard_align=shape.align)
    cap_pages = int(max_pinned_gib * (1 << 30)) // B.host_pool_bytes(one)
    if cap_pages < shape.host_pages:
        log(f"[bench] host pool capped at {cap_pages} of {shape.host_pages} pages ({max_pinned_gib} GiB pinned)")
        shape = W.shape_scaled(shape, shape.name, host_pages=cap_pages)
    return shape


def measure(args):
    """Every measurement of the headline workload; the result dict, or None for the modes that
    print their own line."""
    import numpy as np
    import torch

    from host_device_page_amd import binding as B
    from host_device_page_amd import workloads as W

    shape = W.SHAPES[args.workload]
    L, P = shape.layers, shape.page_size
    shape = capped_shape(B, W, args.workload, args.max_pinned_gib)
    log(f"[bench] workload {shape.name}: L={L} P={P} subs={shape.subs} S={shape.device_slots} H={shape.host_pages}")
    t_setup = time.perf_counter()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2)
    dev = []
    for g, e in shape.subs:
        units = shape.device_slots // P if g == 1 else shape.device_slots
        dev.append(torch.empty((L, units * e), dtype=torch.uint8, device="cuda").random_(0, 256, generator=gen))
    if args.exchange_only:
        # no host pool: the exchange runs on device memory only
        calibration_copy(torch, args.calibration_copy_mib)
        stream = torch.cuda.Stream()
        burst = W.burst_for(shape, seed=1)
        d2 = W.fresh_slots_like(shape, burst, seed=2)
        d2_t = torch.from_numpy(d2).cuda()
        torch.cuda.synchronize()
        log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; exchange of {burst.n} tokens per layer")
        res = layer_exchange_timing(B, np, shape, dev, d2_t, burst.n, stream, counter_workload=shape.name)
        log(f"[bench] layer exchange {res}")
        print(json.dumps({"layer_exchange": res, "workload": shape.name}), flush=True)
        return None
    probe, _k = B.make_desc(layers=L, page_size=P, subs=[(g, e, [1] * L) for g, e in shape.subs],
                            device_slots=shape.device_slots, host_pages=shape.host_pages, layout=shape.layout,
                            shard_align=shape.align)
    host = B.HostBuffer(B.host_pool_bytes(probe))
    stream = torch.cuda.Stream()
    wb_mode = {"auto": B.HC_MODE_AUTO, "zerocopy": B.HC_MODE_ZEROCOPY, "staged": B.HC_MODE_STAGED}[args.write_back_mode]
    staging = None
    if wb_mode == B.HC_MODE_STAGED or not args.no_staged_probe:
        img = B.staging_page_bytes(probe)
        if args.staging_pages <= 0:
            args.staging_pages = max(1, STAGING_CHUNK_BYTES // img)
        staging = torch.empty(args.staging_pages * img, dtype=torch.uint8, device="cuda")
    layers = [[t[l] for l in range(L)] for t in dev]

    def make_pool(mode, max_ctas=None, flags=B.HC_FLAG_PROFILE, stream_=None):
        return B.Pool(layers=L, page_size=P, subs=list(shape.subs), device_slots=shape.device_slots,
                      host_pages=shape.host_pages, device_layers=layers, host=host,
                      stream=stream if stream_ is None else stream_,
                      layout=shape.layout, shard_align=shape.align, staging=staging, write_back_mode=mode,
                      flags=flags, max_ctas=args.max_ctas if max_ctas is None else max_ctas)

    calibration_copy(torch, args.calibration_copy_mib)
    pool = make_pool(wb_mode)
    burst = W.burst_for(shape, seed=1)
    d2 = W.fresh_slots_like(shape, burst, seed=2)
    d_t = torch.from_numpy(burst.device_idx).cuda()
    h_np = np.ascontiguousarray(burst.host_idx)
    h_t = torch.from_numpy(h_np).cuda()
    d2_t = torch.from_numpy(d2).cuda()
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; burst {burst.n} tokens, {burst.pages.size} pages; "
        f"write-back mode {pool.mode(0)} (1 staged, 2 zero-copy), load-back mode {pool.mode(1)}")
    if args.beside_compute:
        pool.close()
        pools = {"zerocopy": make_pool(B.HC_MODE_ZEROCOPY, flags=0), "staged": make_pool(B.HC_MODE_STAGED, flags=0)}
        res = write_back_overlap(B, torch, np, pools, d_t, h_np, consumers=args.compute_streams)
        for p in pools.values():
            p.close()
        print(json.dumps({"beside_compute": res, "workload": shape.name,
                          "burst_bytes_each_way": burst_bytes(shape, burst)[0]}), flush=True)
        host.free()
        return None
    if args.sweep:
        # no per-launch timing events here: at small bursts their cost (~9 us per launch) would dominate
        pool.close()
        pool = make_pool(wb_mode, flags=0)
        rows = burst_size_sweep(B, np, pool, shape, stream, burst, d_t, h_np, h_t, d2_t, args)
        print(json.dumps({"sweep": "burst size", "workload": shape.name, "write_back_mode": pool.mode(0),
                          "max_ctas": args.max_ctas or DEFAULT_MAX_CTAS, "rows": rows}), flush=True)
        pool.close()
        host.free()
        return None

    link_bytes, _ = burst_bytes(shape, burst)
    if args.gather_patterns:
        pool.close()
        rows = gather_patterns(B, torch, np, W, make_pool, shape, burst, h_np, staged_bytes(shape, burst))
        print(json.dumps({"gather_patterns": rows, "workload": shape.name, "chunk_pages": args.staging_pages}),
              flush=True)
        host.free()
        return None
    if args.gather_dram:
        pool.close()
        res = gather_dram_bound(B, torch, np, W, make_pool, stream, shape, burst, args.staging_pages)
        log(f"[bench] gather with nothing in the Infinity Cache: {res}")
        print(json.dumps({"gather_dram_bound": res, "workload": shape.name}), flush=True)
        host.free()
        return None
    if args.duplex_only:
        pool.close()
        hip = hip_setup(B)
        nb = min(1 << 30, host.nbytes // 2 // 4096 * 4096)
        scratch = torch.empty(2 * nb, dtype=torch.uint8, device="cuda")
        res = duplex_measurement(B, torch, np, hip, make_pool, shape, burst, d_t, h_np, d2_t, link_bytes, host,
                                 scratch, nb, args.duplex_pairs, staging is not None)
        del scratch
        print(json.dumps({"duplex": res, "workload": shape.name, "burst_bytes_each_way": link_bytes}), flush=True)
        host.free()
        return None
    ev_wb0, ev_wb1, ev_lb1 = B.HipEvent(timing=True), B.HipEvent(timing=True), B.HipEvent(timing=True)
    layer_events = [B.HipEvent() for _ in range(L)]
    enqueue_s = []

    def step(record):
        t0 = time.perf_counter()
        if record:
            ev_wb0.record(stream)
        pool.write_back_all_layers(d_t, h_np)
        if record:
            ev_wb1.record(stream)
        for l in range(L):
            pool.load_back_layer(l, h_t, d2_t, layer_events[l])
        if record:
            ev_lb1.record(stream)
        enqueue_s.append(time.perf_counter() - t0)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    pool.kernel_time(0, reset=True)
    enqueue_s.clear()
    wb_ms, lb_ms = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        ev_lb1.synchronize()
        wb_ms.append(ev_wb0.elapsed_ms(ev_wb1))
        lb_ms.append(ev_wb1.elapsed_ms(ev_lb1))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {el:.3f} s")
    kinds = {k: pool.kernel_time(k) for k in range(6)}
    pool.sync()
    step_ms = el * 1e3 / args.steps
    value = 2 * link_bytes * args.steps / el / 1e9
    wb_gbs = link_bytes / (float(np.median(wb_ms)) * 1e-3) / 1e9
    lb_gbs = link_bytes / (float(np.median(lb_ms)) * 1e-3) / 1e9

    # host-link peaks measured here: 1 GiB hipMemcpyAsync pinned <-> device, best of 5
    hip = hip_setup(B)
    # 1 GiB, or half the host pool when it is smaller (the copies land in the host pool)
    one_gib = min(1 << 30, host.nbytes // 2 // 4096 * 4096)
    scratch = torch.empty(2 * one_gib, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    peak_h2d = memcpy_peak(hip, host.ptr.value, scratch.data_ptr(), one_gib, stream.cuda_stream, True)
    peak_d2h = memcpy_peak(hip, host.ptr.value, scratch.data_ptr(), one_gib, stream.cuda_stream, False)
    duplex = None
    if not args.no_duplex:
        duplex = duplex_measurement(B, torch, np, hip, make_pool, shape, burst, d_t, h_np, d2_t, link_bytes,
                                    host, scratch, one_gib, args.duplex_pairs, staging is not None)
    del scratch
    log(f"[bench] hipMemcpyAsync peak H2D {peak_h2d:.2f} GB/s, D2H {peak_d2h:.2f} GB/s")

    # dominant kernel: per-launch algorithmic bytes / mean HIP-event launch duration
    n_rd, ms_rd = kinds[B.KIND_ZC_READ]
    n_wr, ms_wr = kinds[B.KIND_ZC_WRITE]
    per_layer_bytes = link_bytes // L
    rd_gbs = per_layer_bytes * n_rd / (ms_rd * 1e-3) / 1e9 if n_rd else None
    wr_gbs = link_bytes * n_wr / (ms_wr * 1e-3) / 1e9 if n_wr else None
    if n_wr and ms_wr > ms_rd:
        dom = {"kernel": "k_zc_write (zero-copy write-back, all layers)", "achieved": wr_gbs, "peak": peak_d2h,
               "launches": n_wr, "avg_ms": ms_wr / n_wr, "bytes_per_launch": link_bytes, "name": "k_zc_write"}
    else:
        dom = {"kernel": "k_zc_read (zero-copy load-back, one layer)", "achieved": rd_gbs, "peak": peak_h2d,
               "launches": n_rd, "avg_ms": ms_rd / max(1, n_rd), "bytes_per_launch": per_layer_bytes,
               "name": "k_zc_read"}
    traffic = counter_traffic(shape.name, dom["name"])
    roofline = {"bound": "host_link", "kernel": dom["kernel"], "achieved": round(dom["achieved"], 3),
                "peak": round(dom["peak"], 3), "unit": "GB/s", "frac": round(dom["achieved"] / dom["peak"], 4),
                "traffic": traffic["bytes"] if traffic else None,
                "traffic_detail": traffic,
                "traffic_algorithmic": 2 * dom["bytes_per_launch"],
                "avg_launch_ms": round(dom["avg_ms"], 4),
                "bytes_per_launch": dom["bytes_per_launch"],
                "peak_source": "hipMemcpyAsync pinned<->device 1 GiB best of 5, measured in this run",
                "peak_published": PCIE5_X16_GBS, "frac_of_published": round(dom["achieved"] / PCIE5_X16_GBS, 4)}
    # layer-wise pipeline: a consumer doing real work per layer, waiting on each layer event
    pipeline = layer_pipeline(B, torch, pool, shape, h_t, d2_t, burst.n, stream, layer_events, make_pool, args)

    # hand-over cost on the calling thread: the per-layer enqueue inline vs on the loader thread,
    # on a pool without per-launch timing (a launch that stamps timing events costs more CPU time)
    handover = {}
    hpool = make_pool(wb_mode, flags=0)
    # CPU time of the enqueue calls alone (validation, planning, plan upload, launches) on this pool
    wb_enq, lb_enq = [], []
    for _ in range(5):
        torch.cuda.synchronize()
        t_s = time.perf_counter()
        hpool.write_back_all_layers(d_t, h_np)
        wb_enq.append(time.perf_counter() - t_s)
        t_s = time.perf_counter()
        for l in range(L):
            hpool.load_back_layer(l, h_t, d2_t, layer_events[l])
        lb_enq.append(time.perf_counter() - t_s)
    hpool.sync()
    enqueue_unprofiled = {"write_back": round(1e3 * float(np.median(wb_enq)), 4),
                          "load_back_all_layers": round(1e3 * float(np.median(lb_enq)), 4)}
    log(f"[bench] CPU enqueue without timing events (ms): {enqueue_unprofiled}")
    for asynchronous in (False, True):
        ld = B.Loader(hpool, L, asynchronous=asynchronous)
        times = []
        for _ in range(5):
            t_s = time.perf_counter()
            bu = ld.submit(h_t, d2_t, burst.n, layer_events)
            times.append(time.perf_counter() - t_s)
            bu.wait()
            bu.release()
        ld.close()
        handover["loader_thread" if asynchronous else "inline"] = round(1e3 * float(np.median(times)), 4)
    # the same burst captured once and handed to the loader thread as a replay
    g_events = [B.HipEvent() for _ in range(L)]
    cap = hpool.capture_load_back(h_t, d2_t, g_events)
    ld = B.Loader(hpool, L, asynchronous=True)
    times = []
    for _ in range(5):
        t_s = time.perf_counter()
        bu = ld.submit_graph(cap, g_events)
        times.append(time.perf_counter() - t_s)
        bu.wait()
        bu.release()
    ld.close()
    cap.close()
    handover["loader_thread_captured"] = round(1e3 * float(np.median(times)), 4)
    graph = load_back_graph_timing(B, np, hpool, stream, L, h_t, d2_t, link_bytes)
    log(f"[bench] captured load-back burst: {graph}")
    hpool.close()
    log(f"[bench] load-back hand-over per burst (ms): {handover}")
    pool.close()
    exchange = layer_exchange_timing(B, np, shape, dev, d2_t, burst.n, stream, counter_workload=shape.name)
    log(f"[bench] layer exchange {exchange}")

    # staged relayout kernel (HBM-bound): same burst through the staged write-back
    roofline_hbm = None
    staged = None
    if not args.no_staged_probe:
        roofline_hbm, staged = staged_probe(B, torch, np, W, make_pool, stream, shape, burst, d_t, h_np, link_bytes,
                                            max(3, args.steps // 2), args.staging_pages)
        # both write-back modes beside independent compute, on pools without timing events
        ov_pools = {"zerocopy": make_pool(B.HC_MODE_ZEROCOPY, flags=0), "staged": make_pool(B.HC_MODE_STAGED, flags=0)}
        staged["beside_compute"] = write_back_overlap(B, torch, np, ov_pools, d_t, h_np)
        for p in ov_pools.values():
            p.close()
        log(f"[bench] staged write-back {staged}")

    cpu = cpu_mt = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle sample ...")
        cpu = cpu_baseline(shape, burst, d2, args.cpu_seconds)
        log(f"[bench] CPU oracle {cpu['value']} GB/s")
        t = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        if t > 1:
            cpu_mt = cpu_baseline(shape, burst, d2, args.cpu_seconds / 2, threads=t)
            log(f"[bench] CPU oracle, {cpu_mt['cores']} threads: {cpu_mt['value']} GB/s")
        exchange["cpu_baseline"] = cpu_exchange_baseline(shape, burst, d2, args.cpu_seconds / 4)
        log(f"[bench] CPU oracle, layer exchange: {exchange['cpu_baseline']['value']} GB/s")

    pages = burst.pages.size
    out = {
        "metric": "write-back/load-back GB/s per burst; % of HBM and host-link peak",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": shape.name, "layers": L, "page_size": P, "row_bytes": list(shape.row_bytes),
                   "device_slots": shape.device_slots, "host_pages": shape.host_pages,
                   "burst_pages": int(pages), "burst_tokens": burst.n,
                   "burst_bytes_each_way": link_bytes, "slots": SLOT_DRAWS.get(shape.name, "seeded random"),
                   "write_back_mode": "staged" if wb_mode == B.HC_MODE_STAGED else "zerocopy",
                   "load_back_mode": "zerocopy"},
        "write_back_GBps": round(wb_gbs, 3), "load_back_GBps": round(lb_gbs, 3),
        "pages_per_s": round(2 * pages * args.steps / el, 1),
        "host_link_peak_GBps": {"h2d": round(peak_h2d, 3), "d2h": round(peak_d2h, 3)},
        "frac_of_link_peak": {"write_back": round(wb_gbs / peak_d2h, 4), "load_back": round(lb_gbs / peak_h2d, 4)},
        "cpu_enqueue_ms_per_step": round(1e3 * float(np.median(enqueue_s)), 3),
        "cpu_enqueue_ms_unprofiled": enqueue_unprofiled,
        "load_back_graph": graph,
        "load_back_handover_ms": handover,
        "layer_pipeline": pipeline,
        "duplex": duplex,
        "kernel_avg_ms": {"zc_read": round(ms_rd / max(1, n_rd), 4), "zc_write": round(ms_wr / max(1, n_wr), 4)},
        "roofline": roofline,
        "roofline_hbm": roofline_hbm,
        "staged_write_back": staged,
        "layer_exchange": exchange,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_mt,
    }
    host.free()
    out["_peaks"] = {"h2d": peak_h2d, "d2h": peak_d2h}
    return out


def main():
    args = parse()
    if args.h2h:
        return h2h_main(args)
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; --gpus above 1 is not supported. The multi-GPU "
                                   "design (layer-owner sharding with a per-layer broadcast) is described, "
                                   "not built."}), flush=True)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    out = measure(args)
    if out is None:
        return
    peaks = out.pop("_peaks")
    if args.second_workload and args.second_workload != args.workload:
        import gc
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["second_workload"] = second_block(args, args.second_workload, peaks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
