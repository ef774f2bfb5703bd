"""fp64 CPU oracle of the L^3 forward and backward passes (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
``static_token_routed_amd`` and imports nothing from it.

* ``forward``: the per-token fp64 loop of ``l3_oracle.c`` (plain C, OpenMP over
  tokens), taking any float inputs widened exactly to fp64.
* ``backward``: the gradients of the same function (chain rule per token,
  parameter gradients summed over tokens), single-threaded fp64 C.
* ``route`` / ``route_bruteforce``: the stable sort by token ID and the per-ID
  blocks (``route.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .route import route, route_bruteforce  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "l3_oracle.c")
LIB = os.path.join(HERE, "libl3oracle.so")

OK, BAD_OFFSETS, TOKEN_RANGE, NOMEM = 0, -2, -3, -6


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", *extra, src, "-o",
           out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_libs: dict = {}


def load(path: str = LIB) -> ctypes.CDLL:
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.l3o_forward.restype = ctypes.c_int
    lib.l3o_forward.argtypes = [I64, I64, I64, ctypes.c_int32, P, I64, I64, I64, I64,
                                P, P, P, P, P, P, P, ctypes.c_double, P, P, P, P, P,
                                ctypes.c_int]
    lib.l3o_backward.restype = ctypes.c_int
    lib.l3o_backward.argtypes = [I64, I64, I64, ctypes.c_int32, P, I64, I64, I64, I64,
                                 P, P, P, P, P, P, P, ctypes.c_double, P, P,
                                 P, P, P, P, P, P, P, P, P]
    lib.l3o_check_offsets.restype = ctypes.c_int
    lib.l3o_check_offsets.argtypes = [P, I64, I64, ctypes.c_int32]
    _libs[path] = lib
    return lib


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__({BAD_OFFSETS: "bad offsets", TOKEN_RANGE: "token id out of range",
                          NOMEM: "out of memory"}.get(code, str(code)))
        self.code = code


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def forward(off, k: int, x, ids, W_K, W_V, W_up, gamma, beta, W_mix, eps: float = 1e-5,
            stages: bool = False, nthreads: int = 0, v: int | None = None,
            lib: ctypes.CDLL | None = None):
    """out [n x d_out] (fp64); with ``stages`` also (o, h, y)."""
    lib = lib or load()
    off = np.ascontiguousarray(off, dtype=np.int64)
    vocab = len(off) - 1
    v = int(off[-1]) if v is None else int(v)
    x, W_K, W_V, W_up, W_mix = map(_f64, (x, W_K, W_V, W_up, W_mix))
    gamma, beta = _f64(gamma), _f64(beta)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = len(ids)
    d_in, d_emb = W_K.shape[1], W_V.shape[1]
    d_up, d_out = W_up.shape[0], W_mix.shape[0]
    assert x.shape == (n, d_in) and W_up.shape == (d_up, d_emb)
    assert W_mix.shape == (d_out, d_up + d_in) and gamma.shape == beta.shape == (d_up,)
    assert W_K.shape[0] == W_V.shape[0]
    out = np.zeros((n, d_out))
    o = np.zeros((n, d_emb)) if stages else None
    h = np.zeros((n, d_up)) if stages else None
    y = np.zeros((n, d_up)) if stages else None
    nul = ctypes.c_void_p(0)
    rc = lib.l3o_forward(n, vocab, v, int(k), _p(off), d_in, d_emb, d_up, d_out,
                         _p(x), _p(ids), _p(W_K), _p(W_V), _p(W_up), _p(gamma), _p(beta),
                         float(eps), _p(W_mix), _p(out),
                         _p(o) if stages else nul, _p(h) if stages else nul,
                         _p(y) if stages else nul, int(nthreads))
    if rc:
        raise OracleError(rc)
    return (out, o, h, y) if stages else out


def backward(off, k: int, x, ids, W_K, W_V, W_up, gamma, beta, W_mix, dout, eps: float = 1e-5,
             v: int | None = None, lib: ctypes.CDLL | None = None, magnitudes: bool = False) -> dict:
    """Gradients of sum(dout * forward(...)) (fp64): dict with dx, dW_K, dW_V, dW_up,
    dgamma, dbeta, dW_mix.  With ``magnitudes`` also kmag and vmag [v]: per table row,
    the size of the products its gradient is formed from (key rows: sum over tokens of
    p_j (||V_j * do||_2 + ||o * do||_2) max|x|, the root sums of squares of the two inner
    products whose difference is dS_j; value rows: sum over tokens of p_j max|do|;
    do = dL/do), zero for rows of absent IDs.  ||dW_V[j]||_inf <= vmag[j]."""
    lib = lib or load()
    off = np.ascontiguousarray(off, dtype=np.int64)
    vocab = len(off) - 1
    v = int(off[-1]) if v is None else int(v)
    x, W_K, W_V, W_up, W_mix, dout = map(_f64, (x, W_K, W_V, W_up, W_mix, dout))
    gamma, beta = _f64(gamma), _f64(beta)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = len(ids)
    d_in, d_emb = W_K.shape[1], W_V.shape[1]
    d_up, d_out = W_up.shape[0], W_mix.shape[0]
    assert x.shape == (n, d_in) and dout.shape == (n, d_out)
    assert W_mix.shape == (d_out, d_up + d_in) and W_up.shape == (d_up, d_emb)
    g = {"dx": np.zeros((n, d_in)), "dW_K": np.zeros((v, d_in)), "dW_V": np.zeros((v, d_emb)),
         "dW_up": np.zeros((d_up, d_emb)), "dgamma": np.zeros(d_up), "dbeta": np.zeros(d_up),
         "dW_mix": np.zeros((d_out, d_up + d_in))}
    rc = lib.l3o_backward(n, vocab, v, int(k), _p(off), d_in, d_emb, d_up, d_out,
                          _p(x), _p(ids), _p(W_K), _p(W_V), _p(W_up), _p(gamma), _p(beta),
                          float(eps), _p(W_mix), _p(dout),
                          *[_p(g[key]) for key in ("dx", "dW_K", "dW_V", "dW_up", "dgamma",
                                                   "dbeta", "dW_mix")],
                          *((_p(g.setdefault("kmag", np.zeros(v))), _p(g.setdefault("vmag", np.zeros(v))))
                            if magnitudes else (ctypes.c_void_p(0), ctypes.c_void_p(0))))
    if rc:
        raise OracleError(rc)
    return g


def check_offsets(off, v: int, k: int, lib: ctypes.CDLL | None = None) -> int:
    lib = lib or load()
    off = np.ascontiguousarray(off, dtype=np.int64)
    return lib.l3o_check_offsets(_p(off), len(off) - 1, int(v), int(k))
