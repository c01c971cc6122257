"""The rank-sharded host tier across processes (rank-sharded tier page, sglang PR 41984,
Accuracy Tests: a multi-process gloo simulation with zero page mismatches, and negative
controls for a skipped exchange and diverging host pages).

Each rank is its own process (tests/rank_shard_worker.py) with its own replica of the
device pool on the one GPU; the owner of a layer packs it after loading and broadcasts
the packed bytes over gloo (CPU tensors), the others unpack them.  Every rank must end
with the oracle's unsharded load-back, the replicas must agree, and the cross-rank page
check must pass; each negative control must be caught."""
import json
import os
import socket
import subprocess
import sys
import time

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
pytestmark = pytest.mark.gpu


def free_port() -> int:
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def run_ranks(world: int, extra_env=None, timeout: float = 240.0):
    port = free_port()
    procs = []
    for r in range(world):
        env = dict(os.environ, RANK=str(r), WORLD_SIZE=str(world), MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port),
                   **(extra_env or {}))
        procs.append(subprocess.Popen([sys.executable, "-u", os.path.join(HERE, "rank_shard_worker.py")], env=env,
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    deadline = time.monotonic() + timeout
    outs = []
    try:
        for p in procs:
            out, err = p.communicate(timeout=max(1.0, deadline - time.monotonic()))
            outs.append((p.returncode, out, err))
    finally:
        for p in procs:
            if p.poll() is None:
                p.kill()
                p.wait()
    results = []
    for r, (rc, out, err) in enumerate(outs):
        assert rc == 0, f"rank {r} exited with {rc}: {err[-3000:]}"
        results.append(json.loads(out.strip().splitlines()[-1]))
    return results


@pytest.mark.timeout(300)
@pytest.mark.parametrize("world", [2, 3, 4])
def test_sharded_tier_over_gloo(world):
    print(f"[rank shard gloo] world {world}", flush=True)
    res = run_ranks(world)
    owned = sorted(l for r in res for l in r["owned"])
    assert owned == list(range(7)), "every layer has exactly one owner"
    for r in res:
        assert r["matches_oracle"], f"rank {r['rank']} differs from the oracle"
        assert r["replicas_agree"] and r["pages_agree"], r


@pytest.mark.timeout(300)
def test_negative_controls_are_caught():
    print("[rank shard gloo] negative controls", flush=True)
    res = run_ranks(3, {"HC_SKIP_RANK": "1"})
    assert all(not r["replicas_agree"] for r in res), "a skipped exchange went unnoticed"
    assert not res[1]["matches_oracle"] and res[0]["matches_oracle"] and res[2]["matches_oracle"]
    res = run_ranks(3, {"HC_DIVERGE_RANK": "2"})
    assert all(not r["pages_agree"] for r in res), "diverging host pages went unnoticed"
