"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` takes a loaded oracle library and raises ``AssertionError`` when
the oracle disagrees with a closed form, an invariant, a special case that
reduces to a library routine, or the pages' second formulation of the layer
(ordinary attention over the whole table with an "allowed rows" mask,
"L^3: Large Lookup Layers", kimjy99.github.io page, section "2. Efficient
Training and Inference").  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires each mistake to fail at least one pin.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed=0, vocab=7, k=5, d_in=6, d_emb=5, d_up=4, d_out=3, n=11, d=None,
          eps=1e-5, gamma_beta=True):
    """Small random problem (fp64 values)."""
    r = _rng(seed)
    if d is None:
        d = r.integers(1, k + 1, size=vocab)
    d = np.asarray(d, np.int64)
    off = np.concatenate([[0], np.cumsum(d)]).astype(np.int64)
    v = int(off[-1])
    ids = r.integers(0, vocab, size=n).astype(np.int32)
    c = dict(off=off, k=k, x=r.standard_normal((n, d_in)), ids=ids,
             W_K=r.standard_normal((v, d_in)) / np.sqrt(d_in),
             W_V=r.standard_normal((v, d_emb)),
             W_up=r.standard_normal((d_up, d_emb)) / np.sqrt(d_emb),
             gamma=1 + 0.5 * r.standard_normal(d_up) if gamma_beta else np.ones(d_up),
             beta=0.5 * r.standard_normal(d_up) if gamma_beta else np.zeros(d_up),
             W_mix=r.standard_normal((d_out, d_up + d_in)) / np.sqrt(d_up + d_in), eps=eps)
    return c


def _run(lib, c, **kw):
    args = dict(c)
    args.update(kw)
    return oracle.forward(args["off"], args["k"], args["x"], args["ids"], args["W_K"],
                          args["W_V"], args["W_up"], args["gamma"], args["beta"],
                          args["W_mix"], eps=args["eps"], stages=True, lib=lib)


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ closed forms

def pin_single_row_slice_is_the_row(lib):
    """d_t = 1: the softmax of one score is exactly 1, so o is the V row, bit for bit."""
    c = _case(1, vocab=6, k=4, d=[1, 3, 1, 2, 1, 4], n=40)
    _, o, _, _ = _run(lib, c)
    for i, t in enumerate(c["ids"]):
        if c["off"][t + 1] - c["off"][t] == 1:
            assert np.array_equal(o[i], c["W_V"][c["off"][t]]), f"token {i}"


def pin_identical_keys_give_mean_of_values(lib):
    """All rows of K_t equal: every score is equal, p_j = 1/d_t, o = mean of V_t."""
    c = _case(2, vocab=5, k=6, d=[3, 6, 2, 5, 4], n=30)
    WK = c["W_K"].copy()
    for t in range(5):
        a, b = c["off"][t], c["off"][t + 1]
        WK[a:b] = WK[a]
    _, o, _, _ = _run(lib, c, W_K=WK)
    for i, t in enumerate(c["ids"]):
        a, b = c["off"][t], c["off"][t + 1]
        _close(o[i], c["W_V"][a:b].mean(0), 1e-14, "mean of V_t")


def pin_zero_state(lib):
    """x = 0: scores are 0 (uniform softmax, o = mean V_t), and the x-columns of
    W_mix cannot matter: out = W_mix[:, :d_up] y."""
    c = _case(3, n=20)
    x0 = np.zeros_like(c["x"])
    out, o, _, y = _run(lib, c, x=x0)
    for i, t in enumerate(c["ids"]):
        a, b = c["off"][t], c["off"][t + 1]
        _close(o[i], c["W_V"][a:b].mean(0), 1e-14, "uniform softmax")
    d_up = c["W_up"].shape[0]
    _close(out, y @ c["W_mix"][:, :d_up].T, 1e-13, "out with x = 0")
    Wm = c["W_mix"].copy()
    Wm[:, d_up:] = _rng(33).standard_normal(Wm[:, d_up:].shape)
    out2, _, _, _ = _run(lib, c, x=x0, W_mix=Wm)
    assert np.array_equal(out, out2), "x-columns of W_mix changed the output at x = 0"


def pin_hand_expanded_two_dims(lib):
    """d_in = d_emb = d_up = 2, d_t in {1, 2, 3}: every stage written out by hand."""
    r = _rng(4)
    d = [1, 2, 3]
    off = np.array([0, 1, 3, 6], np.int64)
    WK, WV = r.standard_normal((6, 2)), r.standard_normal((6, 2))
    Wup, Wmix = r.standard_normal((2, 2)), r.standard_normal((3, 4))
    g, bb = 1 + 0.3 * r.standard_normal(2), 0.3 * r.standard_normal(2)
    x = r.standard_normal((9, 2))
    ids = np.array([0, 1, 2, 2, 1, 0, 2, 1, 2], np.int32)
    eps = 1e-3
    out = oracle.forward(off, 3, x, ids, WK, WV, Wup, g, bb, Wmix, eps=eps, lib=lib)
    import math
    for i, t in enumerate(ids):
        a = int(off[t])
        x0, x1 = x[i]
        s = [WK[a + j, 0] * x0 + WK[a + j, 1] * x1 for j in range(d[t])]
        if d[t] == 1:
            p = [1.0]
        elif d[t] == 2:
            p1 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
            p = [p1, 1.0 - p1]
        else:
            e = [math.exp(s[0]), math.exp(s[1]), math.exp(s[2])]
            p = [e[0] / sum(e), e[1] / sum(e), e[2] / sum(e)]
        o0 = sum(p[j] * WV[a + j, 0] for j in range(d[t]))
        o1 = sum(p[j] * WV[a + j, 1] for j in range(d[t]))
        h0 = Wup[0, 0] * o0 + Wup[0, 1] * o1
        h1 = Wup[1, 0] * o0 + Wup[1, 1] * o1
        half = (h0 - h1) / 2.0              # h - mean for the first feature
        den = math.sqrt(half * half + eps)  # biased variance of two values is half^2
        y0 = half / den * g[0] + bb[0]
        y1 = -half / den * g[1] + bb[1]
        ref = [Wmix[q, 0] * y0 + Wmix[q, 1] * y1 + Wmix[q, 2] * x0 + Wmix[q, 3] * x1
               for q in range(3)]
        _close(out[i], ref, 1e-13, f"hand-expanded token {i}")


def pin_layernorm_closed_form(lib):
    """gamma = 1, beta = 0: mean(y) = 0 and mean(y^2) = var(h) / (var(h) + eps);
    with gamma, beta: y = gamma * y_plain + beta (affine after normalising)."""
    c = _case(5, d_up=7, n=25, eps=1e-2, gamma_beta=False)
    _, _, h, y = _run(lib, c)
    var = h.var(axis=1)                      # numpy biased variance
    _close(y.mean(axis=1), np.zeros(len(y)), 1e-13, "mean(y)")
    _close((y * y).mean(axis=1), var / (var + c["eps"]), 1e-13, "mean(y^2)")
    r = _rng(55)
    g, b = 1 + r.standard_normal(7), r.standard_normal(7)
    _, _, _, y2 = _run(lib, c, gamma=g, beta=b)
    _close(y2, y * g + b, 1e-13, "affine gamma/beta")


# ------------------------------------------------------------------ invariances

def pin_softmax_shift_invariance(lib):
    """Adding one vector u to every row of K_t shifts all d_t scores by <u, x>:
    the softmax, hence the output, does not change."""
    c = _case(6, n=30)
    out, _, _, _ = _run(lib, c)
    WK = c["W_K"].copy()
    r = _rng(66)
    for t in range(len(c["off"]) - 1):
        a, b = c["off"][t], c["off"][t + 1]
        WK[a:b] += r.standard_normal(WK.shape[1])
    out2, _, _, _ = _run(lib, c, W_K=WK)
    _close(out2, out, 1e-12, "shifted keys")


def pin_row_permutation_invariance(lib):
    """Permuting the rows of a slice in K and V together leaves the output unchanged
    (a softmax-weighted sum does not depend on the order of its terms)."""
    c = _case(7, n=30)
    out, _, _, _ = _run(lib, c)
    WK, WV = c["W_K"].copy(), c["W_V"].copy()
    r = _rng(77)
    for t in range(len(c["off"]) - 1):
        a, b = c["off"][t], c["off"][t + 1]
        p = a + r.permutation(b - a)
        WK[a:b], WV[a:b] = c["W_K"][p], c["W_V"][p]
    out2, _, _, _ = _run(lib, c, W_K=WK, W_V=WV)
    _close(out2, out, 1e-12, "permuted slice rows")


def pin_value_scale_invariance(lib):
    """Scaling W_V by alpha > 0 scales o and h by alpha; LayerNorm (eps ~ 0)
    removes it, so y and the output do not change."""
    c = _case(8, n=30, eps=1e-300)
    out, _, _, _ = _run(lib, c)
    out2, _, _, _ = _run(lib, c, W_V=3.5 * c["W_V"])
    _close(out2, out, 1e-12, "scaled values")


def pin_token_independence(lib):
    """The layer mixes channels only: one token alone gives its row of the batched
    result exactly, and shuffling the batch shuffles the rows."""
    c = _case(9, n=24)
    out, _, _, _ = _run(lib, c)
    for i in (0, 7, 23):
        one, _, _, _ = _run(lib, c, x=c["x"][i:i + 1], ids=c["ids"][i:i + 1])
        assert np.array_equal(one[0], out[i]), f"token {i} alone"
    p = _rng(99).permutation(24)
    outp, _, _, _ = _run(lib, c, x=c["x"][p], ids=c["ids"][p])
    assert np.array_equal(outp, out[p]), "shuffled batch"


# ------------------------------------------------------------------ other formulations

def pin_masked_dense_attention(lib):
    """The pages' batch formulation: ordinary attention with Q = X, K = W_K,
    V = W_V over the whole table, every row outside the token's slice masked
    out.  Computed here with dense numpy matrices (no per-token slicing)."""
    cfg = synth.small(vocab=40, k=9, d_in=12, d_emb=10, d_up=8, d_out=6, n=64, v=200)
    off = synth.offsets(cfg)
    c = _case(10, n=64, d_in=12, d_emb=10, d_up=8, d_out=6, vocab=40, k=9,
              d=np.diff(off))
    _, o, _, _ = _run(lib, c)
    S = c["x"] @ c["W_K"].T                                   # n x v
    rows = np.arange(S.shape[1])
    allowed = (rows[None, :] >= c["off"][c["ids"]][:, None]) & \
              (rows[None, :] < c["off"][c["ids"] + 1][:, None])
    S = np.where(allowed, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    _close(o, P @ c["W_V"], 1e-13, "masked dense attention")


def pin_linear_stages_and_identities(lib):
    """The linear stages equal numpy matmuls of the oracle's own stage outputs;
    W_mix = [0 | I] returns x exactly and W_mix = [I | 0] returns y exactly."""
    c = _case(11, d_in=4, d_up=4, d_out=4, n=21)
    out, o, h, y = _run(lib, c)
    _close(h, o @ c["W_up"].T, 1e-14, "h = o W_up^T")
    _close(out, np.concatenate([y, c["x"]], 1) @ c["W_mix"].T, 1e-14, "out = [y x] W_mix^T")
    I, Z = np.eye(4), np.zeros((4, 4))
    o1, _, _, y1 = _run(lib, c, W_mix=np.concatenate([Z, I], 1))
    assert np.array_equal(o1, c["x"]), "W_mix = [0 | I] must return x"
    o2, _, _, y2 = _run(lib, c, W_mix=np.concatenate([I, Z], 1))
    assert np.array_equal(o2, y2), "W_mix = [I | 0] must return y"


def pin_offsets_and_ids_checked(lib):
    """Allocation bounds 1 <= d_t <= k and sum d_t = v are enforced; IDs outside
    [0, vocab) are rejected."""
    good = np.array([0, 2, 3, 7], np.int64)
    assert oracle.check_offsets(good, 7, 4, lib=lib) == 0
    assert oracle.check_offsets(np.array([0, 2, 2, 7], np.int64), 7, 5, lib=lib) != 0  # d = 0
    assert oracle.check_offsets(good, 7, 3, lib=lib) != 0                               # d > k
    assert oracle.check_offsets(good, 8, 4, lib=lib) != 0                               # v
    assert oracle.check_offsets(np.array([1, 2, 3, 7], np.int64), 7, 4, lib=lib) != 0
    c = _case(12, n=5)
    bad = c["ids"].copy()
    bad[2] = len(c["off"]) - 1
    try:
        _run(lib, c, ids=bad)
    except oracle.OracleError as e:
        assert e.code == oracle.TOKEN_RANGE
    else:
        raise AssertionError("out-of-range id accepted")


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
