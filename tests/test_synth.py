"""Seeded input generator: allocation constraints, the pages' hyper-parameters,
reproducibility and row-range regeneration.  CPU only."""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_allocation_constraints(name):
    cfg = synth.CONFIGS[name]
    d = synth.allocation(cfg)
    assert len(d) == cfg.vocab and d.sum() == cfg.v
    assert d.min() >= 1 and d.max() <= cfg.k
    off = synth.offsets(cfg)
    assert off[0] == 0 and off[-1] == cfg.v and np.array_equal(np.diff(off), d)
    ids = synth.token_ids(cfg)
    assert ids.dtype == np.int32 and len(ids) == cfg.n
    assert ids.min() >= 0 and ids.max() < cfg.vocab


def test_paper_config_matches_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    cfg = synth.CONFIGS["paper_bf16"]
    assert (cfg.v, cfg.k, cfg.vocab) == (g["v"], g["k"], g["vocab"])
    assert cfg.n % g["seq_len"] == 0
    d = synth.allocation(cfg)
    # frequent tokens reach the cap, rare ones keep the minimum (Fig. 5 shape)
    assert d[0] == g["k"] and d[-1] == g["min_per_token"]
    assert np.all(np.diff(d) <= 0)            # non-increasing in token rank
    assert cfg.v / cfg.k > g["sparsity_lower_bound"]
    per_tok = d.max() * (cfg.d_in + cfg.d_emb)
    assert 0.5 * g["params_per_token_order"] <= per_tok <= 2 * g["params_per_token_order"]


def test_skew_allocation():
    cfg = synth.CONFIGS["skew_bf16"]
    d = synth.allocation(cfg)
    assert np.all(d[:200] == 512)
    ids = synth.token_ids(cfg)
    assert np.sum(ids < 200) == cfg.n // 2 and np.all(d[ids[ids >= 200]] == 1)
    u = synth.allocation(synth.CONFIGS["skew_uniform_bf16"])
    assert set(np.unique(u)) == {3, 4}


def test_reproducible_and_row_regeneration():
    cfg = synth.small(vocab=50, k=8, d_in=64, d_emb=64, d_up=64, d_out=64, n=9000, v=300,
                      dtype="bf16")
    a = synth.hidden(cfg)
    assert np.array_equal(a, synth.hidden(cfg))
    rows = np.array([0, 4095, 4096, 8999, 17])
    assert np.array_equal(synth.hidden(cfg, rows=rows), a[rows])
    wk = synth.table(cfg, "W_K")
    assert np.array_equal(synth.table(cfg, "W_K", rows=np.array([299, 3])), wk[[299, 3]])
    f = synth.as_f32(wk, "bf16")
    assert abs(f.std() * np.sqrt(64) - 1) < 0.05


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3], np.float32)
    b = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert b.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]   # ties go to even
    assert abs(b[4] - 1e-3) <= 2 ** -9 * 1e-3
