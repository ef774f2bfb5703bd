"""Route oracle (stable sort by token ID and per-ID blocks) against a hand-worked
fixture, the pure-Python brute force and the invariants of a sort.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ["perm", "sorted_ids", "inv_perm", "uniq", "counts", "seg_start"]


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "route_hand.json")))
    for fn in (oracle.route, oracle.route_bruteforce):
        r = fn(np.array(g["ids"], np.int32), g["vocab"])
        for key in KEYS:
            assert r[key].tolist() == g[key], (fn.__name__, key)
        assert r["num_segments"] == g["num_segments"] and r["err"] == g["err"]


@pytest.mark.parametrize("seed,n,vocab", [(0, 1, 3), (1, 50, 4), (2, 300, 1000), (3, 257, 7),
                                          (4, 1000, 1), (5, 0, 10)])
def test_matches_bruteforce(seed, n, vocab):
    ids = np.random.default_rng(seed).integers(-2, vocab + 2, size=n).astype(np.int32)
    a, b = oracle.route(ids, vocab), oracle.route_bruteforce(ids, vocab)
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), key
    assert a["num_segments"] == b["num_segments"] and a["err"] == b["err"]


def test_invariants_large():
    ids = np.random.default_rng(9).integers(0, 180000, size=131072).astype(np.int32)
    r = oracle.route(ids, 180000)
    n = len(ids)
    assert np.array_equal(np.sort(r["perm"]), np.arange(n))          # a permutation
    assert np.all(np.diff(r["sorted_ids"]) >= 0)                      # non-decreasing
    assert np.array_equal(ids[r["perm"]], r["sorted_ids"])
    assert np.array_equal(r["perm"][r["inv_perm"]], np.arange(n))     # inverse
    assert np.all(np.diff(r["uniq"]) > 0) and r["counts"].sum() == n
    assert r["seg_start"][-1] == n and np.array_equal(np.diff(r["seg_start"]), r["counts"])
    # stability: inside a block the batch indices increase
    for s0, s1 in zip(r["seg_start"][:-1][:500], r["seg_start"][1:][:500]):
        assert np.all(np.diff(r["perm"][s0:s1]) > 0)
    assert not r["err"]
