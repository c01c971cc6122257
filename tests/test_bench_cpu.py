"""Host-side pieces of the benchmark, on the CPU: the one-GPU contract, the byte
accounting, the counter lookup's code digest and the slicing of the CPU oracle
sample across threads."""
import json
import os
import subprocess
import sys
import threading

import numpy as np

import bench
from host_device_page_amd import workloads as W
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_burst_bytes_counts_rows_per_layer_and_blocks_per_page():
    shape = W.SHAPES["dsa_mla_indexer_78l"]
    burst = W.burst_for(shape, seed=4)
    link, _ = bench.burst_bytes(shape, burst)
    P, L = shape.page_size, shape.layers
    assert burst.n % P == 0
    assert link == L * (burst.n * 1152 + (burst.n // P) * 8448)
    shape = W.SHAPES["llama3_8b_mha_bf16"]
    burst = W.burst_for(shape, seed=5)
    assert bench.burst_bytes(shape, burst)[0] == shape.layers * burst.n * 2 * 2048 == 2 << 30


def test_kernel_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    base = bench.kernel_source_digest()
    src = open(os.path.join(ROOT, "host_device_page_amd", "csrc", "hc_kernels.hip")).read()
    fake = tmp_path / "host_device_page_amd" / "csrc"
    fake.mkdir(parents=True)
    (fake / "hc_kernels.hip").write_text("// a new comment\n" + src.replace("\n", "\n\n") + "\n/* trailing */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_digest() == base
    (fake / "hc_kernels.hip").write_text(src.replace("HC_TILE", "HC_TILE_X", 1))
    assert bench.kernel_source_digest() != base


def test_counter_traffic_is_dropped_when_the_kernels_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = {"kernels": {"k_zc_write": {"fetch_bytes": 10, "write_bytes": 20}}}
    (prof / "w_counters.json").write_text(json.dumps(dict(entry, kernel_code_digest=bench.kernel_source_digest())))
    (prof / "old_counters.json").write_text(json.dumps(dict(entry, kernel_code_digest="0" * 64)))
    src_dir = tmp_path / "host_device_page_amd" / "csrc"
    src_dir.mkdir(parents=True)
    src_dir.joinpath("hc_kernels.hip").write_text(
        open(os.path.join(ROOT, "host_device_page_amd", "csrc", "hc_kernels.hip")).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("w", "k_zc_write")["bytes"] == 30
    assert bench.counter_traffic("w", "k_zc_read") is None
    assert bench.counter_traffic("old", "k_zc_write") is None
    assert bench.counter_traffic("missing", "k_zc_write") is None


def test_page_cuts_split_only_between_host_pages():
    for name in ["llama3_8b_mha_bf16", "mha_kv_split_shard_bf16", "dsa_mla_indexer_78l"]:
        shape = W.SHAPES[name]
        h = W.burst_for(shape, seed=7).host_idx
        for parts in (1, 2, 3, 8, 16):
            cuts = bench._page_cuts(h, shape.page_size, parts)
            assert cuts[0] == 0 and cuts[-1] == h.size and all(a < b for a, b in zip(cuts, cuts[1:]))
            assert len(cuts) - 1 <= parts
            pages = [set((h[a:b] // shape.page_size).tolist()) for a, b in zip(cuts[:-1], cuts[1:])]
            assert sum(len(p) for p in pages) == len(set((h // shape.page_size).tolist())), name


def test_threaded_oracle_slices_give_the_whole_burst():
    """The threaded CPU sample does the same work as one call over the burst."""
    shape = W.SHAPES["tiny_mha_bf16"]
    g = O.Geometry(shape.layers, shape.page_size, list(shape.subs), shape.host_pages, shape.device_slots,
                   shape.layout, shape.align)
    rng = np.random.default_rng(3)
    dev = [[rng.integers(0, 256, g.device_units(b) * e, dtype=np.uint8) for _ in range(shape.layers)]
           for b, (_, e) in enumerate(shape.subs)]
    burst = W.burst_for(shape, seed=3)
    whole = np.zeros(O.host_pool_bytes(g), dtype=np.uint8)
    O.write_back(g, dev, whole, burst.device_idx, burst.host_idx)
    sliced = np.zeros_like(whole)
    cuts = bench._page_cuts(burst.host_idx, shape.page_size, 4)
    ts = [threading.Thread(target=O.write_back, args=(g, dev, sliced, burst.device_idx[a:b], burst.host_idx[a:b]))
          for a, b in zip(cuts[:-1], cuts[1:])]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert np.array_equal(whole, sliced)


def test_cpu_baseline_reports_threads_and_bytes():
    shape = W.SHAPES["tiny_mha_bf16"]
    burst = W.burst_for(shape, seed=1)
    d2 = W.fresh_slots_like(shape, burst, seed=2)
    one = bench.cpu_baseline(shape, burst, d2, 0.2)
    two = bench.cpu_baseline(shape, burst, d2, 0.2, threads=2)
    assert one["cores"] == 1 and two["cores"] == 2
    assert one["kind"] == two["kind"] == "oracle" and one["value"] > 0 and two["value"] > 0


def test_duplex_load_back_names_the_same_rows_of_other_pages():
    for name in ("llama3_8b_mha_bf16", "dsa_mla_indexer_78l", "mha_kv_split_shard_bf16"):
        shape = W.SHAPES[name]
        P = shape.page_size
        burst = W.burst_for(shape, seed=1)
        h = burst.host_idx
        o = bench.relabel_host_pages(h, P, shape.host_pages)
        assert o.dtype == np.int64 and o.shape == h.shape
        assert np.array_equal(o % P, h % P)  # rows kept, so the byte count is the same
        assert np.intersect1d(o // P, h // P).size == 0  # disjoint host pages
        assert o.min() >= 0 and o.max() < shape.host_pages * P
        # one new page per old page, and distinct old pages get distinct new ones
        pairs = np.unique(np.stack([h // P, o // P]), axis=1)
        assert pairs.shape[1] == np.unique(h // P).size == np.unique(o // P).size
        assert bench.burst_bytes(shape, W.Burst(burst.device_idx, o, W.distinct_pages(o, P)))[0] == \
            bench.burst_bytes(shape, burst)[0]
    # too few pages left
    assert bench.relabel_host_pages(np.arange(48, dtype=np.int64), 16, 5) is None


def test_duplex_pairs_parse():
    assert bench.parse_pairs("staged:16:8,zerocopy:2:10") == (("staged", 16, 8), ("zerocopy", 2, 10))
    import argparse
    import pytest
    with pytest.raises(argparse.ArgumentTypeError):
        bench.parse_pairs("copy:1:1")
