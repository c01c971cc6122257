"""Randomized parity sweep: many small random pools (layers, page size, row and block
sizes, layouts, modes, partial pages, slot patterns, zero-copy grid caps), each
compared byte for byte with the oracle after a write-back and a per-layer load-back."""
import numpy as np
import pytest

from host_device_page_amd import binding as B
from host_device_page_amd import workloads as W
from gpu_support import Rig, cuda_i64, load_back_and_check, say, write_back_and_check


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    L = int(rng.integers(1, 7))
    P = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    layout = int(rng.choice([W.PAGE_FIRST, W.KV_SPLIT_SHARD, W.PAGE_FIRST_TOKEN_MAJOR]))
    nsub = int(rng.integers(1, 5))
    blocks = bool(rng.random() < 0.3)
    subs = []
    for b in range(nsub):
        gran = W.PAGE_BLOCKS if (blocks and b == nsub - 1) else W.TOKEN_ROWS
        subs.append((gran, 16 * int(rng.integers(1, 80))))
    H = int(rng.integers(4, 40))
    S = P * int(rng.integers(H + 8, 4 * H + 16))
    align = int(rng.choice([16, 256, 4096]))
    pages = rng.choice(H, size=int(rng.integers(1, H)), replace=False)
    toks = []
    for p in pages:
        rows = P if (blocks or rng.random() < 0.6) else int(rng.integers(1, P + 1))
        start = 0 if blocks else int(rng.integers(0, P - rows + 1))
        toks.append(p * P + np.arange(start, start + rows))
    h = np.concatenate(toks).astype(np.int64)
    if not blocks and rng.random() < 0.5:
        h = h[rng.permutation(h.size)]
    # room for two disjoint slot sets (write-back slots and fresh load-back slots)
    S = max(S, P * (2 * pages.size + 1))
    shape = W.PoolShape(f"rand{seed}", L, P, tuple(subs), S, H, layout, align)
    if blocks:
        dp = rng.choice(S // P, size=pages.size, replace=False)
        d = (dp[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
        free = np.setdiff1d(np.arange(S // P), dp)
        dp2 = rng.choice(free, size=pages.size, replace=False)
        d2 = (dp2[:, None] * P + np.arange(P)[None, :]).reshape(-1).astype(np.int64)
    else:
        d = rng.choice(S, size=h.size, replace=False).astype(np.int64)
        d2 = rng.choice(np.setdiff1d(np.arange(S), d), size=h.size, replace=False).astype(np.int64)
    mode = B.HC_MODE_STAGED if rng.random() < 0.5 else B.HC_MODE_ZEROCOPY
    staging_pages = int(rng.integers(1, 6))
    # the zero-copy grid cap (0 = the library default) from a stream of its own, so the cases above stay as they were
    max_ctas = int(np.random.default_rng(5000 + seed).choice([0, 0, 1, 2, 3, 5, 8, 16, 33, 64, 256]))
    return shape, d, h, d2, mode, staging_pages, max_ctas


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(600))
def test_random_pool(seed):
    shape, d, h, d2, mode, staging_pages, max_ctas = random_case(seed)
    say(f"[random {seed}] L={shape.layers} P={shape.page_size} subs={shape.subs} layout={shape.layout} "
        f"align={shape.align} n={h.size} mode={mode} max_ctas={max_ctas}")
    rig = Rig(shape, seed=seed, write_back_mode=mode, staging_pages=staging_pages, max_ctas=max_ctas)
    try:
        write_back_and_check(rig, d, h)
        load_back_and_check(rig, h, d2)
        assert rig.pool.round_trip_check(cuda_i64(d), cuda_i64(d2)) == 0
    finally:
        rig.close()
