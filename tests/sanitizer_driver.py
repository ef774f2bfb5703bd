"""Run in a child process with a sanitizer runtime preloaded (see test_host_sanitizers.py).

    python sanitizer_driver.py oracle <sanitized oracle .so>
    python sanitizer_driver.py library <host-sanitized libl3 .so>

`oracle`: every forward and backward pin of the fp64 oracle against the sanitized
build.  `library`: the library's host code on caller input without a GPU -- plan and
dims validation (the rejections return before any device call; a valid plan fails
at its first device allocation), workspace sizing over many batch sizes and dims,
the LZW allocation trie on random and adversarial corpora (checked against the
Python oracle), and argument checks of the other entry points.  Imports no torch."""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path[:0] = [ROOT, HERE]


def run_oracle(path: str) -> None:
    import oracle
    from oracle_backward_pins import BACKWARD_PINS
    from oracle_pins import PINS
    lib = oracle.load(path)
    for pin in PINS + BACKWARD_PINS:
        pin(lib)
        print("pin ok:", pin.__name__, flush=True)


class Dims(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int64), ("d_emb", ctypes.c_int64), ("d_up", ctypes.c_int64),
                ("d_out", ctypes.c_int64), ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


def run_library(path: str) -> None:
    from oracle.lzw import allocate as lzw_oracle
    lib = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.l3_plan.argtypes = [P, I64, I64, ctypes.c_int32, ctypes.POINTER(Dims), ctypes.POINTER(P)]
    lib.l3_workspace_size_dims.restype = ctypes.c_size_t
    lib.l3_workspace_size_dims.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, I64]
    lib.l3_allocate_lzw.argtypes = [P, I64, I64, I64, ctypes.c_int32, P]
    lib.l3_gemm_workspace_size.restype = ctypes.c_size_t
    lib.l3_gemm_workspace_size.argtypes = [I64, I64, I64]
    lib.l3_gemm_bf16.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.l3_strerror.restype = ctypes.c_char_p
    rng = np.random.default_rng(0)

    # plan: bad offsets and dims are rejected on the host
    def plan(off, v, k, dims):
        off = np.ascontiguousarray(off, np.int64)
        h = P()
        return lib.l3_plan(off.ctypes.data, len(off) - 1, v, k, ctypes.byref(dims), ctypes.byref(h))
    good = Dims(256, 128, 256, 256, 1, 1e-5)
    for off, v, k in ([0, 2, 2, 5], 5, 4), ([0, 2, 7, 9], 9, 4), ([1, 2, 3, 5], 5, 4), ([0, 2, 3, 5], 6, 4):
        assert plan(off, v, k, good) == -2
    for dims in (Dims(100, 64, 64, 64, 1, 1e-5), Dims(64, 96, 64, 64, 1, 1e-5), Dims(8192, 64, 64, 64, 1, 1e-5),
                 Dims(64, 64, 64, -1, 1, 1e-5), Dims(64, 64, 64, 64, 7, 1e-5), Dims(64, 64, 64, 64, 1, -1.0)):
        assert plan([0, 2, 3, 5], 5, 4, dims) in (-1, -4)
    # a large valid allocation: validated on the host, then the first device call fails
    d = rng.integers(1, 513, size=100000)
    off = np.concatenate([[0], np.cumsum(d)])
    assert plan(off, int(off[-1]), 512, Dims(2048, 512, 2048, 2048, 1, 1e-5)) in (0, -7)
    print("plan checks ok", flush=True)

    # workspace sizing: positive, non-decreasing in n, for several dims and max_d
    for dims, mx in ((Dims(2048, 512, 2048, 2048, 1, 1e-5), 512), (Dims(4096, 512, 4096, 4096, 1, 1e-5), 512),
                     (Dims(192, 64, 128, 64, 1, 1e-5), 90), (Dims(100, 37, 72, 52, 0, 1e-5), 96)):
        prev = 0
        for n in range(1, 1500, 7):
            s = lib.l3_workspace_size_dims(ctypes.byref(dims), mx, n)
            assert s >= prev > 0 or (prev == 0 and s > 0)
            prev = s
    print("workspace sizing ok", flush=True)

    # LZW allocation on random Zipf corpora with spliced phrases, and edge cases
    def lzw(corpus, vocab, v, k):
        c = np.ascontiguousarray(corpus, np.int32)
        out = np.zeros(vocab + 1, np.int64)
        rc = lib.l3_allocate_lzw(c.ctypes.data if c.size else None, c.size, vocab, v, k, out.ctypes.data)
        return rc, out
    for seed in range(6):
        r = np.random.default_rng(seed)
        vocab = int(r.integers(5, 400))
        base = np.minimum(r.zipf(1.3, size=int(r.integers(1, 20000))) - 1, vocab - 1).astype(np.int32)
        phrase = r.integers(0, vocab, size=5).astype(np.int32)
        corpus = np.concatenate([base[: len(base) // 2], np.tile(phrase, 50), base[len(base) // 2:]])
        k = int(r.integers(1, 64))
        v = int(r.integers(vocab, vocab * k + 1))
        rc, off = lzw(corpus, vocab, v, k)
        try:
            want = lzw_oracle(corpus.tolist(), vocab, v, k)
        except ValueError:
            want = None
        assert (rc == 0) == (want is not None) and rc in (0, -5), (seed, rc)
        if rc == 0:
            assert np.array_equal(np.diff(off), np.asarray(want)), seed
    assert lzw(np.zeros(0, np.int32), 4, 4, 2)[0] in (0, -1, -5)
    assert lzw(np.array([0, 5], np.int32), 3, 3, 2)[0] == -3          # token out of range
    assert lzw(np.array([0, 1, 0, 1], np.int32), 2, 9, 2)[0] == -1    # v > vocab * k
    print("lzw ok", flush=True)

    # other entry points: argument checks on the host
    assert lib.l3_gemm_workspace_size(64, 8192, 2048) == 8 * 64 * 8192 * 4
    a, b, c, w = P(0x1000), P(0x2000), P(0x3000), P(0x4000)
    assert lib.l3_gemm_bf16(a, b, c, 64, 64, 96, w, 1 << 30, None) == -4
    assert lib.l3_gemm_bf16(P(0x1008), b, c, 64, 64, 64, w, 1 << 30, None) == -1
    assert lib.l3_gemm_bf16(a, b, c, 64, 8192, 2048, w, 16, None) == -5
    for code in range(-8, 1):
        assert lib.l3_strerror(code)
    print("argument checks ok", flush=True)


if __name__ == "__main__":
    {"oracle": run_oracle, "library": run_library}[sys.argv[1]](sys.argv[2])
    print("SANITIZER_DRIVER_OK", flush=True)
