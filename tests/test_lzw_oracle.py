"""The LZW allocation oracle against the hand-worked example and invariants (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import lzw

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lzw_hand.json")))


def test_codewords_match_hand_derivation():
    got = lzw.codewords(GOLD["corpus"])
    want = {tuple(cw): f for cw, f in GOLD["codewords"]}
    assert got == want


@pytest.mark.parametrize("case", GOLD["cases"], ids=[f"v{c['v']}_k{c['k']}" for c in GOLD["cases"]])
def test_allocation_matches_hand_derivation(case):
    assert lzw.allocate(GOLD["corpus"], GOLD["vocab"], case["v"], case["k"]) == case["d"]


def test_invariants_on_zipf_corpus():
    rng = np.random.default_rng(0)
    vocab, k = 200, 16
    w = 1.0 / np.arange(1, vocab + 1)
    corpus = rng.choice(vocab, size=20000, p=w / w.sum())
    for v in (vocab, 900, 2500, vocab * k):
        d = lzw.allocate(corpus, vocab, v, k)
        assert sum(d) == v and min(d) >= 1 and max(d) <= k
    # frequent tokens get more embeddings than rare ones (the pages' Fig. 5 shape)
    d = lzw.allocate(corpus, vocab, 1500, k)
    assert np.mean(d[:10]) > np.mean(d[-50:])


def test_single_token_corpus_and_bounds():
    # one repeated token: codewords (0,0), (0,0,0), ... all end in token 0
    d = lzw.allocate([0] * 50, 4, 10, 7)
    assert d == [7, 1, 1, 1]
    with pytest.raises(ValueError):
        lzw.allocate([0] * 50, 4, 3, 7)      # v < vocab
    with pytest.raises(ValueError):
        lzw.allocate([0] * 50, 4, 29, 7)     # v > vocab * k
    with pytest.raises(ValueError):
        lzw.allocate([0] * 50, 4, 11, 7)     # token 0 full, no codeword ends elsewhere


# ---- the library's native allocation against the oracle (host code: no GPU needed)

def _lib():
    return pytest.importorskip("static_token_routed_amd")


def _zipf_corpus(seed, vocab, n, s=1.1, phrases=True):
    """Zipf tokens, with repeated phrases spliced in so longer codewords recur."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, vocab + 1) ** s
    base = rng.choice(vocab, size=n, p=w / w.sum()).astype(np.int32)
    if phrases:
        pool = [rng.choice(vocab, size=rng.integers(2, 6), p=w / w.sum()) for _ in range(30)]
        for i in range(0, n - 8, 23):
            ph = pool[rng.integers(0, len(pool))]
            base[i:i + len(ph)] = ph
    return base


@pytest.mark.parametrize("seed,vocab,n,v,k", [(1, 50, 3000, 400, 16), (2, 300, 40000, 5000, 64),
                                              (3, 1000, 120000, 9000, 512), (4, 7, 500, 7, 3)])
def test_native_allocation_matches_oracle(seed, vocab, n, v, k):
    l3 = _lib()
    corpus = _zipf_corpus(seed, vocab, n)
    want = lzw.allocate(corpus, vocab, v, k)
    off = l3.l3_allocate_lzw(corpus, vocab, v, k)
    assert off[0] == 0 and off[-1] == v
    assert np.array_equal(np.diff(off), np.asarray(want, np.int64))


def test_native_allocation_hand_example_and_errors():
    l3 = _lib()
    for case in GOLD["cases"]:
        off = l3.l3_allocate_lzw(GOLD["corpus"], GOLD["vocab"], case["v"], case["k"])
        assert list(np.diff(off)) == case["d"]
    for args, code in [(([0] * 50, 4, 3, 7), l3.L3_ERR_INVALID_ARG), (([0] * 50, 4, 29, 7), l3.L3_ERR_INVALID_ARG),
                       (([0] * 50, 4, 11, 7), l3.L3_ERR_CAPACITY), (([0, 9], 4, 8, 7), l3.L3_ERR_TOKEN_RANGE)]:
        with pytest.raises(l3.L3Error) as e:
            l3.l3_allocate_lzw(*args)
        assert e.value.code == code
