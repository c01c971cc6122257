"""Seeded synthetic workloads for the KV page transfer: pool shapes and index lists.

This module only draws inputs.  It holds none of the transfer arithmetic (no
host or device offsets, no copies), so both the GPU path and the oracle can be
fed from it.  Every generator takes an explicit seed and is deterministic.

The shapes follow the models the pages name: a Llama-3-8B-like MHA pool and a
DeepSeek-V3-like MLA latent pool (hybrid-pool write-back page: MHA, MLA and
DSA indexer pools), a 78-layer MLA model with a second DSA indexer-K host pool
loaded in the same burst (loader-thread page, Motivation; rank-sharded host
tier page, Modifications), and the CacheStore shard layout K page | V page |
pad (CacheStore H2H page, section "page_first_kv_split support").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TOKEN_ROWS = 0
PAGE_BLOCKS = 1
PAGE_FIRST = 0
KV_SPLIT_SHARD = 1
PAGE_FIRST_TOKEN_MAJOR = 2


@dataclass(frozen=True)
class PoolShape:
    """Geometry of one KV pool pair (device layer-first, host page-first or shard)."""

    name: str
    layers: int
    page_size: int
    subs: tuple  # ((granularity, bytes per token row or page block), ...)
    device_slots: int
    host_pages: int
    layout: int = PAGE_FIRST
    align: int = 4096
    sub_names: tuple = field(default=())

    @property
    def row_bytes(self) -> tuple:
        return tuple(e for _, e in self.subs)


def bf16_row_bytes(heads: int, head_dim: int) -> int:
    return heads * head_dim * 2


# DSA indexer page block: 64 fp8-e4m3 keys of 128 bytes, then 64 fp32 scales.
DSA_INDEXER_PAGE_BLOCK = 64 * 128 + 64 * 4

SHAPES = {
    # 4 layers, 8 KV heads x 64 dims bf16, 16-token pages, 4096 slots, 256 host pages.
    "tiny_mha_bf16": PoolShape("tiny_mha_bf16", 4, 16,
                               ((TOKEN_ROWS, bf16_row_bytes(8, 64)),) * 2, 4096, 256,
                               sub_names=("k", "v")),
    # Llama-3-8B: 32 layers, 8 KV heads x 128 dims bf16, 64-token pages.
    "llama3_8b_mha_bf16": PoolShape("llama3_8b_mha_bf16", 32, 64,
                                    ((TOKEN_ROWS, bf16_row_bytes(8, 128)),) * 2, 262144, 8192,
                                    sub_names=("k", "v")),
    # DeepSeek-V3 MLA latent: 61 layers, 512 latent + 64 rope dims bf16, one buffer.
    "dsv3_mla_bf16": PoolShape("dsv3_mla_bf16", 61, 64, ((TOKEN_ROWS, 576 * 2),), 524288, 16384,
                               sub_names=("latent",)),
    # 78-layer MLA + DSA indexer-K pool, loaded in one burst.
    "dsa_mla_indexer_78l": PoolShape("dsa_mla_indexer_78l", 78, 64,
                                     ((TOKEN_ROWS, 576 * 2), (PAGE_BLOCKS, DSA_INDEXER_PAGE_BLOCK)),
                                     524288, 2048, sub_names=("latent", "indexer")),
    # Llama-3-8B pool with the token-major page-first host layout [page][row][layer].
    "llama3_8b_mha_bf16_token_major": PoolShape("llama3_8b_mha_bf16_token_major", 32, 64,
                                                ((TOKEN_ROWS, bf16_row_bytes(8, 128)),) * 2, 262144, 8192,
                                                layout=PAGE_FIRST_TOKEN_MAJOR, sub_names=("k", "v")),
    # MHA in K page | V page | pad shards: 48 layers, 8 x 128 bf16, 32-token pages.
    "mha_kv_split_shard_bf16": PoolShape("mha_kv_split_shard_bf16", 48, 32,
                                         ((TOKEN_ROWS, bf16_row_bytes(8, 128)),) * 2, 262144, 4096,
                                         layout=KV_SPLIT_SHARD, sub_names=("k", "v")),
}


@dataclass
class Burst:
    """One transfer burst: token-granular int64 device slots and host token indices."""

    device_idx: np.ndarray  # int64 [n]
    host_idx: np.ndarray    # int64 [n]; page = h // P, row = h % P
    pages: np.ndarray       # distinct host pages named, in order of first use

    @property
    def n(self) -> int:
        return int(self.device_idx.size)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def host_pages(seed: int, host_page_count: int, k: int) -> np.ndarray:
    """k distinct host pages, uniformly at random."""
    return _rng(seed).choice(host_page_count, size=k, replace=False).astype(np.int64)


def whole_page_tokens(pages: np.ndarray, page_size: int) -> np.ndarray:
    """Host token indices of every row of each page, page by page."""
    return (pages[:, None] * page_size + np.arange(page_size, dtype=np.int64)[None, :]).reshape(-1)


def permutation_slots(seed: int, slots: int, n: int, exclude: np.ndarray | None = None) -> np.ndarray:
    """First n entries of a seeded permutation of the free slots."""
    free = np.ones(slots, dtype=bool)
    if exclude is not None:
        free[exclude] = False
    cand = np.flatnonzero(free)
    if cand.size < n:
        raise ValueError("not enough free slots")
    return _rng(seed).permutation(cand)[:n].astype(np.int64)


def segment_slots(seed: int, slots: int, n: int, p_run: float = 0.5, max_run: int = 64,
                  exclude: np.ndarray | None = None) -> np.ndarray:
    """Free-list draw: each segment is, with probability p_run, a run of U{1..max_run}
    consecutive free slots from a random free start, else one random free slot.
    Slots stay distinct; the list stops at n entries."""
    rng = _rng(seed)
    free = np.ones(slots, dtype=bool)
    if exclude is not None:
        free[exclude] = False
    out = np.empty(n, dtype=np.int64)
    k = 0
    while k < n:
        want = int(rng.integers(1, max_run + 1)) if rng.random() < p_run else 1
        want = min(want, n - k)
        # random free start: rejection draw, falling back to a scan when the pool is dense
        s = -1
        for _ in range(64):
            c = int(rng.integers(0, slots))
            if free[c]:
                s = c
                break
        if s < 0:
            cand = np.flatnonzero(free)
            if cand.size == 0:
                raise ValueError("not enough free slots")
            s = int(cand[rng.integers(0, cand.size)])
        e = s
        while e < slots and e - s < want and free[e]:
            e += 1
        out[k:k + e - s] = np.arange(s, e, dtype=np.int64)
        free[s:e] = False
        k += e - s
    return out


def page_aligned_slots(seed: int, slots: int, page_size: int, n_pages: int,
                       exclude_pages: np.ndarray | None = None) -> np.ndarray:
    """Whole device pages: n_pages distinct random page-aligned blocks, all rows in order."""
    dev_pages = slots // page_size
    free = np.ones(dev_pages, dtype=bool)
    if exclude_pages is not None:
        free[exclude_pages] = False
    cand = np.flatnonzero(free)
    pick = _rng(seed).permutation(cand)[:n_pages].astype(np.int64)
    return whole_page_tokens(pick, page_size)


def scattered_slots(seed: int, slots: int, n: int, exclude: np.ndarray | None = None) -> np.ndarray:
    """Fully random distinct slots with no two list neighbours in adjacent slots."""
    rng = _rng(seed)
    d = permutation_slots(seed, slots, n, exclude)
    for _ in range(1000):
        bad = np.flatnonzero(np.abs(np.diff(d)) == 1) + 1
        if bad.size == 0:
            return d
        for i in bad:
            j = int(rng.integers(0, n))
            d[i], d[j] = d[j], d[i]
    raise RuntimeError("could not separate adjacent slots")


def partial_page_requests(seed: int, host_page_count: int, page_size: int, total_pages: int,
                          max_pages: int = 8) -> np.ndarray:
    """Host token indices for requests of U{1..max_pages} distinct random pages whose
    last page holds U{1..P-1} leading rows, until total_pages pages are named."""
    rng = _rng(seed)
    pages = rng.choice(host_page_count, size=total_pages, replace=False).astype(np.int64)
    toks = []
    k = 0
    while k < total_pages:
        m = min(int(rng.integers(1, max_pages + 1)), total_pages - k)
        for j in range(m):
            rows = page_size if j < m - 1 else int(rng.integers(1, page_size))
            toks.append(pages[k + j] * page_size + np.arange(rows, dtype=np.int64))
        k += m
    return np.concatenate(toks)


def distinct_pages(host_idx: np.ndarray, page_size: int) -> np.ndarray:
    pg = host_idx // page_size
    _, first = np.unique(pg, return_index=True)
    return pg[np.sort(first)]


def burst_for(shape: PoolShape, seed: int, purpose: str = "write_back") -> Burst:
    """The burst a workload moves.  purpose: 'write_back' or 'load_back'."""
    P, S, H = shape.page_size, shape.device_slots, shape.host_pages
    if shape.name == "tiny_mha_bf16":
        pages = host_pages(seed, H, 32)
        h = whole_page_tokens(pages, P)
        d = permutation_slots(seed + 1, S, h.size)
    elif shape.name in ("llama3_8b_mha_bf16", "llama3_8b_mha_bf16_token_major"):
        pages = host_pages(seed, H, 256)
        h = whole_page_tokens(pages, P)
        d = segment_slots(seed + 1, S, h.size)
    elif shape.name == "dsv3_mla_bf16":
        pages = host_pages(seed, H, 512)
        h = whole_page_tokens(pages, P)
        d = segment_slots(seed + 1, S, h.size)
    elif shape.name == "dsa_mla_indexer_78l":
        pages = host_pages(seed, H, 1024)
        h = whole_page_tokens(pages, P)
        d = page_aligned_slots(seed + 1, S, P, pages.size)
    elif shape.name == "mha_kv_split_shard_bf16":
        h = partial_page_requests(seed, H, P, 2048)
        d = scattered_slots(seed + 1, S, h.size)
    else:
        raise KeyError(shape.name)
    return Burst(d, h, distinct_pages(h, P))


def fresh_slots_like(shape: PoolShape, burst: Burst, seed: int) -> np.ndarray:
    """Device slots for a load-back of the same host tokens into slots the burst did
    not use, drawn the way the workload draws its slots."""
    P, S = shape.page_size, shape.device_slots
    n = burst.n
    if any(g == PAGE_BLOCKS for g, _ in shape.subs):
        used_pages = np.unique(burst.device_idx // P)
        return page_aligned_slots(seed, S, P, n // P, exclude_pages=used_pages)
    if shape.name in ("llama3_8b_mha_bf16", "llama3_8b_mha_bf16_token_major", "dsv3_mla_bf16"):
        return segment_slots(seed, S, n, exclude=burst.device_idx)
    if shape.name == "mha_kv_split_shard_bf16":
        return scattered_slots(seed, S, n, exclude=burst.device_idx)
    return permutation_slots(seed, S, n, exclude=burst.device_idx)


def shape_scaled(shape: PoolShape, name: str, *, layers=None, device_slots=None, host_pages=None) -> PoolShape:
    """The same rows and pages with fewer layers or slots (small parity cases)."""
    return PoolShape(name, layers or shape.layers, shape.page_size, shape.subs,
                     device_slots or shape.device_slots, host_pages or shape.host_pages,
                     shape.layout, shape.align, shape.sub_names)
