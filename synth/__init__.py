"""Seeded synthetic inputs for the Large Lookup Layer (L^3) forward pass.

This module only *draws* inputs: allocations, token-ID streams, tables, dense
weights and hidden states.  It holds none of the layer's arithmetic (no
softmax, projection, normalisation, sort or segment logic), so that the fp64
oracle and the GPU path can both be fed from it without sharing any code of
the method itself.

Recipe (every number below is a workload choice, not a fact of the pages):

* RNG: ``numpy.random.PCG64`` seeded by ``SeedSequence(seed, spawn_key=key)``.
  Each tensor has its own key; row-chunked tensors use ``(tensor, chunk)`` so
  any row range can be regenerated on its own (chunk = ``CHUNK_ROWS`` rows).
* Weights ``W ~ N(0, std = 1/sqrt(fan_in))``, fan_in = row length
  (W_K: d_in, W_V: d_emb, W_up: d_emb, W_mix: d_up+d_in).  Hidden states
  ``x ~ N(0, 1)``.  Draws are fp32; bf16 workloads round them to nearest-even
  bf16 and store the 16-bit patterns (``uint16``).
* Allocation D ("Zipf-shaped"): weights ``w_i = (i+1)^-s`` over token IDs
  (lower ID = more frequent = more embeddings, the shape of the pages'
  embedding-count histogram, "L^3: Large Lookup Layers", Fig. 5), water-filled:
  the largest ``c`` with ``sum clip(floor(c*w_i), 1, k) <= v``, then the few
  leftover units go one each to unclipped IDs by descending fractional part
  (ties to the lower ID).  ``sum D = v`` and ``1 <= d_t <= k`` always hold.
* Token streams: truncated Zipf ``P(i) ~ (i+1)^-s`` over ``[0, vocab)`` by
  inverse CDF on uniform draws.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 4096

# Tensor keys of the SeedSequence spawn tree.
KEY_WK, KEY_WV, KEY_WUP, KEY_WMIX, KEY_X, KEY_IDS, KEY_GAMMA, KEY_BETA = range(8)
KEY_PRE_A, KEY_PRE_B = 8, 9


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    vocab: int
    v: int
    k: int
    d_in: int
    d_emb: int
    d_up: int
    d_out: int
    n: int
    dtype: str = "bf16"          # "f32" or "bf16"
    alloc: str = "zipf"          # "zipf" | "skew" | "uniform"
    alloc_s: float = 1.0
    ids: str = "zipf"            # "zipf" | "skew"
    ids_s: float = 1.1
    seed: int = 0
    ln_eps: float = 1e-5
    tied: bool = False           # W_V is W_K (needs d_emb == d_in)
    # decode workload only
    steps: int = 0
    pre_m: int = 0
    pre_k: int = 0
    pre_n: int = 0


CONFIGS = {
    # correctness config, fp32 end to end
    "tiny_f32": Config("tiny_f32", vocab=512, v=2048, k=32, d_in=64, d_emb=64,
                       d_up=64, d_out=64, n=256, dtype="f32", ids_s=1.1),
    "small_bf16": Config("small_bf16", vocab=32000, v=131072, k=128, d_in=1024,
                         d_emb=256, d_up=1024, d_out=1024, n=8 * 2048, ids_s=1.1),
    # the pages' layer size: v = 710K embeddings, k = 512, 180K vocab, 2048 context
    "paper_bf16": Config("paper_bf16", vocab=180000, v=710000, k=512, d_in=2048,
                         d_emb=512, d_up=2048, d_out=2048, n=16 * 2048, ids_s=1.05),
    # decode: small_bf16's tables in pinned host memory, 64 tokens per step
    "decode_bf16": Config("decode_bf16", vocab=32000, v=131072, k=128, d_in=1024,
                          d_emb=256, d_up=1024, d_out=1024, n=64, ids_s=1.05,
                          steps=256, pre_m=64, pre_k=2048, pre_n=8192),
    # the tied variant (W_V = W_K, one table read for both roles): d_in = d_emb = 512
    "tied_bf16": Config("tied_bf16", vocab=180000, v=710000, k=512, d_in=512, d_emb=512,
                        d_up=2048, d_out=2048, n=16 * 2048, ids_s=1.05, tied=True),
    # the same dims with separate tables, for comparison
    "untied512_bf16": Config("untied512_bf16", vocab=180000, v=710000, k=512, d_in=512,
                             d_emb=512, d_up=2048, d_out=2048, n=16 * 2048, ids_s=1.05),
    "skew_bf16": Config("skew_bf16", vocab=180000, v=710000, k=512, d_in=4096,
                        d_emb=512, d_up=4096, d_out=4096, n=64 * 2048,
                        alloc="skew", ids="skew"),
    "skew_uniform_bf16": Config("skew_uniform_bf16", vocab=180000, v=710000, k=512,
                                d_in=4096, d_emb=512, d_up=4096, d_out=4096,
                                n=64 * 2048, alloc="uniform", ids="skew"),
}


def nthreads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


# ---------------------------------------------------------------- bf16 codec

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to nearest-even bf16, return the 16-bit patterns (no NaNs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (fp32 or bf16 bits) -> exact fp32 values."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


# ---------------------------------------------------------------- allocation

def waterfill(w: np.ndarray, total: int, lo: int, hi: int) -> np.ndarray:
    """Integer allocation ``d`` with ``lo <= d_i <= hi`` and ``sum d = total``
    shaped like ``c * w``: the largest c with ``sum clip(floor(c w), lo, hi) <= total``,
    then leftover units to unclipped entries by descending fractional part."""
    w = np.asarray(w, dtype=np.float64)
    m = len(w)
    if not (m * lo <= total <= m * hi):
        raise ValueError("budget outside [m*lo, m*hi]")

    def f(c: float) -> int:
        return int(np.clip(np.floor(c * w), lo, hi).sum())

    c_lo, c_hi = 0.0, (hi + 1.0) / float(w.min())
    for _ in range(200):
        mid = 0.5 * (c_lo + c_hi)
        if mid == c_lo or mid == c_hi:
            break
        if f(mid) <= total:
            c_lo = mid
        else:
            c_hi = mid
    cw = c_lo * w
    d = np.clip(np.floor(cw), lo, hi).astype(np.int64)
    rem = total - int(d.sum())
    if rem:
        frac = cw - np.floor(cw)
        idx = np.arange(m)
        elig = idx[(d < hi) & (cw >= lo)]
        order = elig[np.lexsort((elig, -frac[elig]))]
        if len(order) < rem:  # pathological ties: fall back to any entry below hi
            extra = idx[(d < hi) & ~np.isin(idx, order)]
            order = np.concatenate([order, extra])
        d[order[:rem]] += 1
    assert int(d.sum()) == total and d.min() >= lo and d.max() <= hi
    return d


def allocation(cfg: Config) -> np.ndarray:
    """D = (d_t) for t in [0, vocab): int64, 1 <= d_t <= k, sum = v."""
    if cfg.alloc == "zipf":
        w = np.arange(1, cfg.vocab + 1, dtype=np.float64) ** (-cfg.alloc_s)
        return waterfill(w, cfg.v, 1, cfg.k)
    if cfg.alloc == "skew":
        forced = 200
        rest = cfg.v - forced * cfg.k
        w = np.arange(forced + 1, cfg.vocab + 1, dtype=np.float64) ** (-cfg.alloc_s)
        return np.concatenate([np.full(forced, cfg.k, np.int64), waterfill(w, rest, 1, cfg.k)])
    if cfg.alloc == "uniform":
        hi = -(-cfg.v // cfg.vocab)           # ceil(v / vocab)
        n_hi = cfg.v - (hi - 1) * cfg.vocab   # IDs that get the larger count
        d = np.full(cfg.vocab, hi - 1, np.int64)
        d[:n_hi] = hi
        assert int(d.sum()) == cfg.v
        return d
    raise ValueError(cfg.alloc)


def offsets(cfg: Config) -> np.ndarray:
    """CSR offsets off[0..vocab] (int64) of the allocation: rows of token t are
    [off[t], off[t+1]) in W_K and W_V."""
    d = allocation(cfg)
    off = np.zeros(cfg.vocab + 1, np.int64)
    np.cumsum(d, out=off[1:])
    return off


# ---------------------------------------------------------------- token streams

def zipf_ids(vocab: int, s: float, n: int, rng: np.random.Generator) -> np.ndarray:
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    cdf[-1] = 1.0
    return np.searchsorted(cdf, rng.random(n), side="right").astype(np.int32)


def token_ids(cfg: Config, n: int | None = None, step: int | None = None) -> np.ndarray:
    """Token IDs (int32).  ``step`` selects an independent stream per decode step."""
    n = cfg.n if n is None else n
    rng = _rng(cfg.seed, KEY_IDS) if step is None else _rng(cfg.seed, KEY_IDS, step)
    if cfg.ids == "zipf":
        return zipf_ids(cfg.vocab, cfg.ids_s, n, rng)
    if cfg.ids == "skew":
        # half of the tokens uniform over the 200 forced IDs, half uniform over the
        # IDs that hold one embedding in the skewed allocation; then shuffled
        d = allocation(dataclasses.replace(cfg, alloc="skew"))
        ones = np.flatnonzero(d == 1)
        h = n // 2
        a = rng.integers(0, 200, size=h)
        b = ones[rng.integers(0, len(ones), size=n - h)]
        return rng.permutation(np.concatenate([a, b])).astype(np.int32)
    raise ValueError(cfg.ids)


# ---------------------------------------------------------------- tensors

def _chunked_normal(seed: int, key: int, rows: int, cols: int, std: float,
                    dtype: str, row_sel: np.ndarray | None = None,
                    sub: tuple = ()) -> np.ndarray:
    """Rows of an N(0, std) matrix drawn chunk by chunk (CHUNK_ROWS rows per chunk,
    each chunk its own stream), optionally only the rows in ``row_sel``."""
    std32 = np.float32(std)
    out_dtype = np.uint16 if dtype == "bf16" else np.float32

    def chunk(j: int) -> np.ndarray:
        r0 = j * CHUNK_ROWS
        nr = min(CHUNK_ROWS, rows - r0)
        a = _rng(seed, key, *sub, j).standard_normal((nr, cols), dtype=np.float32)
        a *= std32
        return _store(a, dtype)

    if row_sel is None:
        out = np.empty((rows, cols), out_dtype)
        nch = -(-rows // CHUNK_ROWS)

        def fill(j: int) -> None:
            r0 = j * CHUNK_ROWS
            out[r0:r0 + CHUNK_ROWS] = chunk(j)

        if nch == 1:
            fill(0)
        else:
            with ThreadPoolExecutor(nthreads()) as ex:
                list(ex.map(fill, range(nch)))
        return out
    row_sel = np.asarray(row_sel, dtype=np.int64)
    out = np.empty((len(row_sel), cols), out_dtype)
    chunks = np.unique(row_sel // CHUNK_ROWS)
    for j in chunks:
        c = chunk(int(j))
        m = (row_sel // CHUNK_ROWS) == j
        out[m] = c[row_sel[m] - j * CHUNK_ROWS]
    return out


def table(cfg: Config, which: str, rows: np.ndarray | None = None) -> np.ndarray:
    """W_K (v x d_in) or W_V (v x d_emb), or only the given rows of it.  A tied
    configuration's W_V is its W_K."""
    if which == "W_V" and cfg.tied:
        return table(cfg, "W_K", rows)
    if which == "W_K":
        return _chunked_normal(cfg.seed, KEY_WK, cfg.v, cfg.d_in, cfg.d_in ** -0.5, cfg.dtype, rows)
    if which == "W_V":
        return _chunked_normal(cfg.seed, KEY_WV, cfg.v, cfg.d_emb, cfg.d_emb ** -0.5, cfg.dtype, rows)
    raise ValueError(which)


def dense(cfg: Config, which: str) -> np.ndarray:
    """W_up (d_up x d_emb) or W_mix (d_out x (d_up + d_in)), torch Linear layout."""
    if which == "W_up":
        return _chunked_normal(cfg.seed, KEY_WUP, cfg.d_up, cfg.d_emb, cfg.d_emb ** -0.5, cfg.dtype)
    if which == "W_mix":
        fan = cfg.d_up + cfg.d_in
        return _chunked_normal(cfg.seed, KEY_WMIX, cfg.d_out, fan, fan ** -0.5, cfg.dtype)
    raise ValueError(which)


def hidden(cfg: Config, n: int | None = None, rows: np.ndarray | None = None,
           step: int | None = None) -> np.ndarray:
    """x ~ N(0, 1), n x d_in (or only the given rows)."""
    n = cfg.n if n is None else n
    sub = () if step is None else (step,)
    return _chunked_normal(cfg.seed, KEY_X, n, cfg.d_in, 1.0, cfg.dtype, rows, sub)


def ln_params(cfg: Config, random: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """LayerNorm gamma, beta (fp32, d_up).  The workloads use gamma=1, beta=0;
    ``random=True`` draws gamma ~ 1 + N(0, 0.5), beta ~ N(0, 0.5) for tests."""
    if not random:
        return np.ones(cfg.d_up, np.float32), np.zeros(cfg.d_up, np.float32)
    g = 1.0 + 0.5 * _rng(cfg.seed, KEY_GAMMA).standard_normal(cfg.d_up, dtype=np.float32)
    b = 0.5 * _rng(cfg.seed, KEY_BETA).standard_normal(cfg.d_up, dtype=np.float32)
    return g.astype(np.float32), b.astype(np.float32)


def pre_gemm_operands(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Decode workload's synthetic pre-layer GEMM operands: A (pre_m x pre_k) and
    B stored as (pre_n x pre_k) (Linear layout), both bf16 N(0, 1/sqrt(pre_k))."""
    std = cfg.pre_k ** -0.5
    a = _chunked_normal(cfg.seed, KEY_PRE_A, cfg.pre_m, cfg.pre_k, std, "bf16")
    b = _chunked_normal(cfg.seed, KEY_PRE_B, cfg.pre_n, cfg.pre_k, std, "bf16")
    return a, b


def small(name: str = "t", *, vocab: int, k: int, d_in: int, d_emb: int, d_up: int,
          d_out: int, n: int, v: int | None = None, dtype: str = "f32", seed: int = 0,
          alloc: str = "zipf", ids_s: float = 1.1, alloc_s: float = 1.0) -> Config:
    """A small ad-hoc configuration for tests."""
    if v is None:
        v = min(vocab * k, max(vocab, 4 * vocab))
    return Config(name, vocab=vocab, v=v, k=k, d_in=d_in, d_emb=d_emb, d_up=d_up,
                  d_out=d_out, n=n, dtype=dtype, alloc=alloc, alloc_s=alloc_s,
                  ids_s=ids_s, seed=seed)
