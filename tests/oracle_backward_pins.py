"""Pins of the fp64 oracle's backward pass against facts that do not come from it.

The gradient of the scalar sum(dout * forward(...)) is pinned against central
finite differences of the oracle's forward pass (itself pinned by
``oracle_pins.py``), and against exact special cases: rows of IDs absent from
the batch get no gradient; with one row per ID the softmax is constant, so the
key rows get none and dx is W2^T dout alone; the gradient is linear in dout.
``test_oracle_backward.py`` runs these pins on the oracle and
``test_oracle_mutants.py`` on copies of it with planted mistakes.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle_pins import _case

KEYS = ("dx", "dW_K", "dW_V", "dW_up", "dgamma", "dbeta", "dW_mix")
ARGS = {"dx": "x", "dW_K": "W_K", "dW_V": "W_V", "dW_up": "W_up", "dgamma": "gamma",
        "dbeta": "beta", "dW_mix": "W_mix"}


def _bwd(lib, c, dout):
    return oracle.backward(c["off"], c["k"], c["x"], c["ids"], c["W_K"], c["W_V"], c["W_up"],
                           c["gamma"], c["beta"], c["W_mix"], dout, eps=c["eps"], lib=lib)


def _loss(lib, c, dout, **kw):
    a = dict(c)
    a.update(kw)
    out = oracle.forward(a["off"], a["k"], a["x"], a["ids"], a["W_K"], a["W_V"], a["W_up"],
                         a["gamma"], a["beta"], a["W_mix"], eps=a["eps"], lib=lib)
    return float(np.sum(out * dout))


def _fd_check(lib, c, seed, tol=1e-6):
    dout = np.random.default_rng(seed).standard_normal((len(c["ids"]), c["W_mix"].shape[0]))
    g = _bwd(lib, c, dout)
    for key in KEYS:
        arr = c[ARGS[key]]
        fd = np.zeros_like(arr, dtype=np.float64)
        for idx in np.ndindex(arr.shape):
            e = 1e-6 * max(1.0, abs(float(arr[idx])))
            a1, a2 = arr.astype(np.float64).copy(), arr.astype(np.float64).copy()
            a1[idx] += e
            a2[idx] -= e
            fd[idx] = (_loss(lib, c, dout, **{ARGS[key]: a1}) -
                       _loss(lib, c, dout, **{ARGS[key]: a2})) / (2 * e)
        err = float(np.max(np.abs(fd - g[key]))) / max(1e-9, float(np.max(np.abs(fd))))
        assert err <= tol, f"{key}: finite-difference rel err {err:.2e}"


def pin_bwd_finite_differences(lib):
    # several rows per ID (softmax over up to 5 rows), random gamma / beta, repeated IDs
    _fd_check(lib, _case(seed=21, vocab=4, k=5, d_in=4, d_emb=3, d_up=5, d_out=3, n=7), 1)
    # mixed one-row and many-row IDs, d_up small (LayerNorm over 3 features)
    _fd_check(lib, _case(seed=22, vocab=5, k=4, d_in=3, d_emb=4, d_up=3, d_out=4, n=6,
                         d=[1, 4, 2, 1, 3]), 2)


def pin_bwd_untouched_rows_zero(lib):
    # the touched IDs own several rows (with one row the keys get no gradient)
    c = _case(seed=23, vocab=6, k=3, n=5, d=[2, 3, 1, 2, 2, 3])
    c["ids"] = np.array([1, 4, 1, 1, 4], np.int32)
    g = _bwd(lib, c, np.random.default_rng(3).standard_normal((5, c["W_mix"].shape[0])))
    off = c["off"]
    for t in range(6):
        rows = slice(off[t], off[t + 1])
        touched = t in (1, 4)
        for key in ("dW_K", "dW_V"):
            assert (np.any(g[key][rows] != 0)) == touched, f"{key} rows of ID {t}"


def pin_bwd_single_row_slices(lib):
    c = _case(seed=24, vocab=5, k=3, n=8, d=[1, 1, 1, 1, 1])
    dout = np.random.default_rng(4).standard_normal((8, c["W_mix"].shape[0]))
    g = _bwd(lib, c, dout)
    d_up = c["W_up"].shape[0]
    assert np.all(g["dW_K"] == 0), "one row per ID: the keys get no gradient"
    np.testing.assert_allclose(g["dx"], dout @ c["W_mix"][:, d_up:], rtol=1e-12, atol=1e-12)


def pin_bwd_linear_in_dout(lib):
    c = _case(seed=25, vocab=4, k=4, n=6)
    dout = np.random.default_rng(5).standard_normal((6, c["W_mix"].shape[0]))
    g1, g2 = _bwd(lib, c, dout), _bwd(lib, c, 2.0 * dout)
    for key in KEYS:
        assert np.array_equal(2.0 * g1[key], g2[key]), key


def _bwd_mag(lib, c, dout):
    return oracle.backward(c["off"], c["k"], c["x"], c["ids"], c["W_K"], c["W_V"], c["W_up"],
                           c["gamma"], c["beta"], c["W_mix"], dout, eps=c["eps"], lib=lib,
                           magnitudes=True)


def pin_bwd_magnitudes_rows(lib):
    # rows of absent IDs have zero magnitude, touched rows a positive one; a value row's
    # gradient sum_i p_j do_i is at most sum_i p_j max|do_i| (triangle inequality); both
    # magnitudes are linear in dout
    c = _case(seed=26, vocab=6, k=4, n=9, d=[3, 1, 4, 2, 2, 4])
    c["ids"] = np.array([0, 2, 2, 5, 0, 1, 2, 5, 0], np.int32)
    dout = np.random.default_rng(6).standard_normal((9, c["W_mix"].shape[0]))
    g = _bwd_mag(lib, c, dout)
    g3 = _bwd_mag(lib, c, 3.0 * dout)
    off = c["off"]
    for t in range(6):
        rows = slice(off[t], off[t + 1])
        present = t in (0, 1, 2, 5)
        for mag in ("kmag", "vmag"):
            m = g[mag][rows]
            assert np.all(m > 0) == present and (present or np.all(m == 0)), (mag, t)
            np.testing.assert_allclose(g3[mag][rows], 3.0 * m, rtol=1e-12)
        assert np.all(np.max(np.abs(g["dW_V"][rows]), axis=1) <= g["vmag"][rows] * (1 + 1e-12))


def pin_bwd_magnitudes_closed_form(lib):
    # one token whose ID owns three rows: its value-row gradients are p_j * do, so
    # do = dW_V[j] / p_j; with p = softmax(K_t x) and o = V_t^T p (three numbers, worked
    # here in numpy) the magnitudes are p_j (||V_j * do||_2 + ||o * do||_2) max|x| and
    # p_j max|do|.  A one-row ID (p = 1, o = V) gives 2 ||V * do||_2 max|x|.
    for d, tok in (([3, 1], 0), ([3, 1], 1)):
        c = _case(seed=27, vocab=2, k=3, n=1, d=d)
        c["ids"] = np.array([tok], np.int32)
        g = _bwd_mag(lib, c, np.random.default_rng(7).standard_normal((1, c["W_mix"].shape[0])))
        a, b = c["off"][tok], c["off"][tok + 1]
        s = c["W_K"][a:b] @ c["x"][0]
        p = np.exp(s - s.max())
        p /= p.sum()
        do = g["dW_V"][a] / p[0]
        V = c["W_V"][a:b]
        o = p @ V
        xmax = np.max(np.abs(c["x"][0]))
        for j in range(b - a):
            want_k = p[j] * (np.linalg.norm(V[j] * do) + np.linalg.norm(o * do)) * xmax
            want_v = p[j] * np.max(np.abs(do))
            np.testing.assert_allclose(g["kmag"][a + j], want_k, rtol=1e-12)
            np.testing.assert_allclose(g["vmag"][a + j], want_v, rtol=1e-12)
        if b - a == 1:
            np.testing.assert_allclose(g["kmag"][a], 2 * np.linalg.norm(V[0] * do) * xmax,
                                       rtol=1e-12)


BACKWARD_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_bwd_")]
