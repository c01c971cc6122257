"""Seeded input generators: distinctness, ranges, run statistics, partial pages (CPU only)."""
import numpy as np
import pytest

from host_device_page_amd import workloads as W


def runs(d):
    """Lengths of maximal runs of consecutive slots."""
    if d.size == 0:
        return np.array([], dtype=np.int64)
    brk = np.flatnonzero(np.diff(d) != 1) + 1
    edges = np.concatenate([[0], brk, [d.size]])
    return np.diff(edges)


def test_segment_slots_distinct_and_mixed():
    d = W.segment_slots(7, 262144, 16384)
    assert d.size == 16384 and np.unique(d).size == d.size
    assert d.min() >= 0 and d.max() < 262144
    r = runs(d)
    # half the segments are runs of U{1..64}, so long runs exist and singletons dominate
    assert r.max() > 32 and (r == 1).mean() > 0.3
    assert np.array_equal(d, W.segment_slots(7, 262144, 16384)), "not deterministic"


def test_scattered_slots_have_no_adjacent_neighbours():
    d = W.scattered_slots(3, 262144, 40000)
    assert np.unique(d).size == d.size
    assert not np.any(np.abs(np.diff(d)) == 1)


def test_page_aligned_slots_are_whole_pages():
    d = W.page_aligned_slots(5, 524288, 64, 1024)
    assert d.size == 1024 * 64 and np.unique(d).size == d.size
    pg = d.reshape(-1, 64)
    assert np.all(pg[:, 0] % 64 == 0)
    assert np.all(np.diff(pg, axis=1) == 1)


def test_partial_page_requests():
    h = W.partial_page_requests(11, 4096, 32, 2048)
    assert np.unique(h).size == h.size
    pages = W.distinct_pages(h, 32)
    assert pages.size == 2048
    counts = np.bincount(h // 32, minlength=4096)[pages]
    assert np.all(counts >= 1) and np.all(counts <= 32)
    assert (counts < 32).sum() > 100, "partial last pages missing"
    # every page's rows are a prefix 0..k-1
    for p in pages[:200]:
        rows = np.sort(h[h // 32 == p] % 32)
        assert np.array_equal(rows, np.arange(rows.size))


@pytest.mark.parametrize("name", ["tiny_mha_bf16", "llama3_8b_mha_bf16", "dsv3_mla_bf16",
                                  "dsa_mla_indexer_78l", "mha_kv_split_shard_bf16"])
def test_bursts(name):
    s = W.SHAPES[name]
    b = W.burst_for(s, seed=1)
    assert b.device_idx.dtype == np.int64 and b.host_idx.dtype == np.int64
    assert np.unique(b.device_idx).size == b.n and np.unique(b.host_idx).size == b.n
    assert b.device_idx.max() < s.device_slots and b.host_idx.max() < s.host_pages * s.page_size
    fresh = W.fresh_slots_like(s, b, seed=2)
    assert fresh.size == b.n and np.unique(fresh).size == b.n
    assert np.intersect1d(fresh, b.device_idx).size == 0
    expect_pages = {"tiny_mha_bf16": 32, "llama3_8b_mha_bf16": 256, "dsv3_mla_bf16": 512,
                    "dsa_mla_indexer_78l": 1024, "mha_kv_split_shard_bf16": 2048}[name]
    assert b.pages.size == expect_pages
