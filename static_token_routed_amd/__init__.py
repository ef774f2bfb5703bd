"""Python binding of libl3.so, the MI355X L^3 forward library (include/l3.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and streams; tensors are passed as raw
pointers.  The functions keep the C names (``l3_plan``, ``l3_forward``, ...);
``L3Plan`` and ``Staging`` wrap them for convenience.  Importing fails loudly
when the library has not been built (``__graft_entry__.build()``): there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libl3.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc, gfx950); there is no CPU fallback")
# torch bundles its own HIP runtime with the same SONAME (libamdhip64.so.7) as the
# system one libl3.so links against; whichever is loaded first serves the whole
# process.  Loading torch first makes libl3.so bind to torch's runtime, so device
# pointers and streams from torch are valid in the library's calls.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

L3_OK, L3_ERR_INVALID_ARG, L3_ERR_BAD_OFFSETS, L3_ERR_TOKEN_RANGE = 0, -1, -2, -3
L3_ERR_UNSUPPORTED, L3_ERR_CAPACITY, L3_ERR_NOMEM, L3_ERR_HIP = -4, -5, -6, -7
L3_F32, L3_BF16 = 0, 1

_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class l3_dims_t(ctypes.Structure):
    _fields_ = [("d_in", _I64), ("d_emb", _I64), ("d_up", _I64), ("d_out", _I64),
                ("dtype", _I32), ("ln_eps", ctypes.c_float)]


_SIG = {
    "l3_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "l3_plan": (ctypes.c_int, [_P, _I64, _I64, _I32, ctypes.POINTER(l3_dims_t), ctypes.POINTER(_P)]),
    "l3_plan_destroy": (ctypes.c_int, [_P]),
    "l3_plan_info": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "l3_worklist_rule": (ctypes.c_int, [_P, _P, _P]),
    "l3_workspace_size": (_SZ, [_P, _I64]),
    "l3_workspace_size_dims": (_SZ, [ctypes.POINTER(l3_dims_t), _I32, _I64]),
    "l3_forward": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "l3_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "l3_backward_workspace_size": (_SZ, [_P, _I64]),
    "l3_allocate_lzw": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int32, _P]),
    "l3_staging_set_cache": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P]),
    "l3_staging_stats": (ctypes.c_int, [_P, _P, _P]),
    "l3_backward": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, _P, _SZ, _P]),
    "l3_route": (ctypes.c_int, [_P, _P, _I64, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P]),
    "l3_status": (ctypes.c_int, [_P, _P]),
    "l3_staging_create": (ctypes.c_int, [_P, _I64, _I64, ctypes.POINTER(_P)]),
    "l3_staging_destroy": (ctypes.c_int, [_P]),
    "l3_prefetch": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P, _P, _P]),
    "l3_forward_staged": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "l3_gemm_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "l3_gemm_bf16": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "l3_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "l3_profile_read": (ctypes.c_int, [_P, _P, ctypes.c_int]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args

EXPORTS = tuple(_SIG)


class L3Error(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        super().__init__(f"{where}: {l3_strerror(code)} ({code})")
        self.code = code


def _check(rc: int, where: str) -> None:
    if rc != L3_OK:
        raise L3Error(rc, where)


def _ptr(t) -> int | None:
    """Device/host address of a tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ C names

def l3_strerror(code: int) -> str:
    return _lib.l3_strerror(code).decode()


def l3_plan(offsets: np.ndarray, vocab: int, v: int, k: int, d_in: int, d_emb: int, d_up: int,
            d_out: int, dtype: str = "bf16", ln_eps: float = 1e-5) -> int:
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    dims = l3_dims_t(d_in, d_emb, d_up, d_out, L3_BF16 if dtype == "bf16" else L3_F32, ln_eps)
    h = _P()
    _check(_lib.l3_plan(offsets.ctypes.data, vocab, v, k, ctypes.byref(dims), ctypes.byref(h)), "l3_plan")
    return h.value


def l3_plan_destroy(plan: int) -> None:
    _check(_lib.l3_plan_destroy(plan), "l3_plan_destroy")


def l3_plan_info(plan: int) -> dict:
    vocab, v, mx = _I64(), _I64(), _I32()
    k = _I32()
    _check(_lib.l3_plan_info(plan, ctypes.addressof(vocab), ctypes.addressof(v),
                             ctypes.addressof(k), ctypes.addressof(mx)), "l3_plan_info")
    return {"vocab": vocab.value, "v": v.value, "k": k.value, "max_d": mx.value}


def l3_worklist_rule(plan) -> tuple[int, int]:
    """(min_tokens, min_rows): blocks with at least this many tokens or rows run on
    the matrix-core gather-attention (INT32_MAX: no such path for these dims)."""
    mt, mr = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.l3_worklist_rule(plan, ctypes.byref(mt), ctypes.byref(mr)), "l3_worklist_rule")
    return mt.value, mr.value


def l3_workspace_size(plan: int, n_max: int) -> int:
    return int(_lib.l3_workspace_size(plan, n_max))


def l3_workspace_size_dims(d_in: int, d_emb: int, d_up: int, d_out: int, dtype: str, max_d: int,
                           n_max: int, ln_eps: float = 1e-5) -> int:
    dims = l3_dims_t(d_in, d_emb, d_up, d_out, L3_BF16 if dtype == "bf16" else L3_F32, ln_eps)
    return int(_lib.l3_workspace_size_dims(ctypes.byref(dims), max_d, n_max))


def l3_forward(plan, x, token_ids, n, W_K, W_V, W_up, ln_gamma, ln_beta, W_mix, out, workspace,
               workspace_bytes, stream=None) -> None:
    _check(_lib.l3_forward(plan, _ptr(x), _ptr(token_ids), n, _ptr(W_K), _ptr(W_V), _ptr(W_up),
                           _ptr(ln_gamma), _ptr(ln_beta), _ptr(W_mix), _ptr(out), _ptr(workspace),
                           workspace_bytes, _stream(stream)), "l3_forward")


def l3_forward_noalloc(plan, x, token_ids, n, W_K, W_V, W_up, ln_gamma, ln_beta, W_mix, out,
                       stream=None) -> None:
    _check(_lib.l3_forward_noalloc(plan, _ptr(x), _ptr(token_ids), n, _ptr(W_K), _ptr(W_V),
                                   _ptr(W_up), _ptr(ln_gamma), _ptr(ln_beta), _ptr(W_mix),
                                   _ptr(out), _stream(stream)), "l3_forward_noalloc")


def l3_allocate_lzw(corpus, vocab: int, v: int, k: int) -> np.ndarray:
    """CSR offsets (int64 [vocab + 1]) of the LZW-style allocation of v embeddings."""
    c = np.ascontiguousarray(corpus, dtype=np.int32)
    off = np.zeros(vocab + 1, dtype=np.int64)
    _check(_lib.l3_allocate_lzw(c.ctypes.data if c.size else None, c.size, vocab, v, k,
                                off.ctypes.data), "l3_allocate_lzw")
    return off


def l3_backward_workspace_size(plan: int, n_max: int) -> int:
    return int(_lib.l3_backward_workspace_size(plan, n_max))


def l3_backward(plan, x, token_ids, n, W_K, W_V, W_up, ln_gamma, ln_beta, W_mix, dout, dx, dW_K,
                dW_V, dW_up, dln_gamma, dln_beta, dW_mix, workspace, workspace_bytes,
                stream=None) -> None:
    _check(_lib.l3_backward(plan, _ptr(x), _ptr(token_ids), n, _ptr(W_K), _ptr(W_V), _ptr(W_up),
                            _ptr(ln_gamma), _ptr(ln_beta), _ptr(W_mix), _ptr(dout), _ptr(dx),
                            _ptr(dW_K), _ptr(dW_V), _ptr(dW_up), _ptr(dln_gamma), _ptr(dln_beta),
                            _ptr(dW_mix), _ptr(workspace), workspace_bytes, _stream(stream)),
           "l3_backward")


def l3_route(plan, token_ids, n, workspace, workspace_bytes, stream=None, perm=None,
             sorted_ids=None, inv_perm=None, uniq=None, counts=None, seg_start=None,
             num_segments=None) -> None:
    _check(_lib.l3_route(plan, _ptr(token_ids), n, _ptr(workspace), workspace_bytes,
                         _stream(stream), _ptr(perm), _ptr(sorted_ids), _ptr(inv_perm), _ptr(uniq),
                         _ptr(counts), _ptr(seg_start), _ptr(num_segments)), "l3_route")


def l3_status(workspace, stream=None) -> int:
    return _lib.l3_status(_ptr(workspace), _stream(stream))


def l3_staging_create(plan: int, max_rows: int, max_tokens: int) -> int:
    h = _P()
    _check(_lib.l3_staging_create(plan, max_rows, max_tokens, ctypes.byref(h)), "l3_staging_create")
    return h.value


def l3_staging_destroy(staging: int) -> None:
    _check(_lib.l3_staging_destroy(staging), "l3_staging_destroy")


def l3_prefetch(plan, token_ids_host: np.ndarray, n, W_K_host, W_V_host, staging, side_stream,
                ready_event=None) -> None:
    ids = np.ascontiguousarray(token_ids_host, dtype=np.int32)
    ev = None
    if ready_event is not None:
        if not ready_event.cuda_event:
            # torch creates events lazily: give this one a handle (the library
            # records it again after its copies)
            ready_event.record(side_stream)
        ev = ready_event.cuda_event
    _check(_lib.l3_prefetch(plan, ids.ctypes.data, n, _ptr(W_K_host), _ptr(W_V_host), staging,
                            _stream(side_stream), ev), "l3_prefetch")


def l3_staging_set_cache(staging, hot_ids, W_K_host, W_V_host, stream=None) -> None:
    ids = np.ascontiguousarray(hot_ids, dtype=np.int32)
    _check(_lib.l3_staging_set_cache(staging, ids.ctypes.data if ids.size else None, ids.size,
                                     _ptr(W_K_host), _ptr(W_V_host), _stream(stream)),
           "l3_staging_set_cache")


def l3_staging_stats(staging) -> tuple[int, int]:
    rows, cached = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.l3_staging_stats(staging, ctypes.byref(rows), ctypes.byref(cached)), "l3_staging_stats")
    return rows.value, cached.value


def l3_forward_staged(staging, x, n, W_up, ln_gamma, ln_beta, W_mix, out, workspace,
                      workspace_bytes, stream=None) -> None:
    _check(_lib.l3_forward_staged(staging, _ptr(x), n, _ptr(W_up), _ptr(ln_gamma), _ptr(ln_beta),
                                  _ptr(W_mix), _ptr(out), _ptr(workspace), workspace_bytes,
                                  _stream(stream)), "l3_forward_staged")


def l3_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(_lib.l3_gemm_workspace_size(M, N, K))


def l3_gemm_bf16(A, B, C, M, N, K, workspace=None, workspace_bytes=None, stream=None) -> None:
    """C = A B^T; allocates the split-K workspace (torch device memory) when none is given."""
    if workspace is None and l3_gemm_workspace_size(M, N, K) > 0:
        import torch
        workspace = torch.empty(l3_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.l3_gemm_bf16(_ptr(A), _ptr(B), _ptr(C), M, N, K, _ptr(workspace), workspace_bytes,
                             _stream(stream)), "l3_gemm_bf16")


def l3_profile_enable(enable: bool) -> None:
    _check(_lib.l3_profile_enable(int(bool(enable))), "l3_profile_enable")


def l3_profile_read(stages: int = 6) -> tuple[list, list]:
    ms = (ctypes.c_double * stages)()
    cnt = (ctypes.c_int64 * stages)()
    _check(_lib.l3_profile_read(ctypes.addressof(ms), ctypes.addressof(cnt), stages), "l3_profile_read")
    return list(ms), list(cnt)


# ------------------------------------------------------------------ convenience

class L3Plan:
    """A plan plus a reusable workspace (torch device memory)."""

    def __init__(self, offsets, k: int, d_in: int, d_emb: int, d_up: int, d_out: int,
                 dtype: str = "bf16", ln_eps: float = 1e-5, v: int | None = None):
        offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.vocab = len(offsets) - 1
        self.v = int(offsets[-1]) if v is None else int(v)
        self.k, self.dtype = k, dtype
        self.d_in, self.d_emb, self.d_up, self.d_out = d_in, d_emb, d_up, d_out
        self.handle = l3_plan(offsets, self.vocab, self.v, k, d_in, d_emb, d_up, d_out, dtype, ln_eps)
        self._ws = None

    def workspace(self, n: int):
        import torch
        need = l3_workspace_size(self.handle, n)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._ws

    def forward(self, x, ids, W_K, W_V, W_up, gamma, beta, W_mix, out=None, stream=None):
        import torch
        n = ids.numel()
        if out is None:
            out = torch.empty((n, self.d_out), dtype=x.dtype, device=x.device)
        ws = self.workspace(n)
        l3_forward(self.handle, x, ids, n, W_K, W_V, W_up, gamma, beta, W_mix, out, ws,
                   ws.numel(), stream)
        return out

    def route(self, ids, stream=None) -> dict:
        import torch
        n = ids.numel()
        ws = self.workspace(n)
        r = {k: torch.empty(n + (1 if k == "seg_start" else 0), dtype=torch.int32, device=ids.device)
             for k in ("perm", "sorted_ids", "inv_perm", "uniq", "counts", "seg_start")}
        r["num_segments"] = torch.zeros(1, dtype=torch.int32, device=ids.device)
        l3_route(self.handle, ids, n, ws, ws.numel(), stream, **r)
        return r

    def status(self, stream=None) -> int:
        return l3_status(self._ws, stream) if self._ws is not None else L3_OK

    def close(self) -> None:
        if self.handle:
            l3_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DecodeLayers:
    """Decode steps through several lookup layers whose tables stay in pinned host
    memory (the pages' offloaded inference: sciencestack.ai page, Fig. 4 caption;
    papernotes.org page, section 关键设计 item 3, where the layers sit after several
    decoder layers so the row copies hide behind them).

    Each layer has its own plan, staging, side stream and ready event.  ``prefetch``
    is called once when a step's token IDs are known and issues every layer's copy
    at once, each on its own side stream, so layer i's rows move while the main
    stream runs everything before layer i.  ``forward(i, x)`` makes the stream wait
    for layer i's copy and runs its staged forward; layer i + 1 may take layer i's
    output as its input.  Steps can follow each other without host synchronisation:
    the library orders each prefetch after the staged forward that last read its
    staging.  This class only schedules: every step is one C call above.

    layers: list of dicts with keys plan (L3Plan), W_K_host, W_V_host (pinned host
    tensors), W_up, gamma, beta, W_mix (device tensors); max_tokens: tokens per step.
    """

    def __init__(self, layers, max_tokens: int):
        import torch
        self.max_tokens = max_tokens
        self.layers = []
        for spec in layers:
            plan = spec["plan"]
            lay = dict(spec)
            lay["staging"] = l3_staging_create(plan.handle, max_tokens * plan.k, max_tokens)
            lay["side"] = torch.cuda.Stream()
            lay["ready"] = torch.cuda.Event()
            lay["ws"] = torch.empty(l3_workspace_size(plan.handle, max_tokens), dtype=torch.uint8,
                                    device="cuda")
            dt = torch.bfloat16 if plan.dtype == "bf16" else torch.float32
            lay["out"] = torch.empty((max_tokens, plan.d_out), dtype=dt, device="cuda")
            self.layers.append(lay)
        self.n = 0

    def set_cache(self, i: int, hot_ids, stream=None) -> None:
        lay = self.layers[i]
        l3_staging_set_cache(lay["staging"], hot_ids, lay["W_K_host"], lay["W_V_host"], stream)

    def stats(self, i: int) -> tuple[int, int]:
        return l3_staging_stats(self.layers[i]["staging"])

    def prefetch(self, token_ids_host) -> None:
        """Issue every layer's row copy for this step's IDs (host int32 [n])."""
        ids = np.ascontiguousarray(token_ids_host, dtype=np.int32)
        self.n = len(ids)
        for lay in self.layers:
            l3_prefetch(lay["plan"].handle, ids, self.n, lay["W_K_host"], lay["W_V_host"],
                        lay["staging"], lay["side"], lay["ready"])

    def forward(self, i: int, x, stream=None):
        """Layer i's output [n x d_out] for input x [n x d_in] (a view of a buffer the
        next step overwrites)."""
        import torch
        lay = self.layers[i]
        s = torch.cuda.current_stream() if stream is None else stream
        s.wait_event(lay["ready"])
        out = lay["out"][: self.n]
        l3_forward_staged(lay["staging"], x, self.n, lay["W_up"], lay["gamma"], lay["beta"],
                          lay["W_mix"], out, lay["ws"], lay["ws"].numel(), s)
        return out

    def close(self) -> None:
        for lay in self.layers:
            if lay.get("staging"):
                l3_staging_destroy(lay["staging"])
                lay["staging"] = 0
