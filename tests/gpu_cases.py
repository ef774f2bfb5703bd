"""Shared helpers of the GPU tests: seeded cases, upload, the library call, and the
fp64 oracle on the same inputs (all tokens, or a sample with the tables reduced to
the sampled IDs' rows)."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

BF16_TOL = 2e-2   # max over rows of ||y - y_ref||_inf / ||y_ref||_inf, bf16 workloads
F32_TOL = 1e-5    # the same for fp32 workloads


@dataclasses.dataclass
class Case:
    cfg: synth.Config
    off: np.ndarray
    ids: np.ndarray
    x: np.ndarray
    WK: np.ndarray
    WV: np.ndarray
    Wup: np.ndarray
    Wmix: np.ndarray
    gamma: np.ndarray
    beta: np.ndarray

    @property
    def tol(self) -> float:
        return BF16_TOL if self.cfg.dtype == "bf16" else F32_TOL

    def f32(self, a):
        return synth.as_f32(a, self.cfg.dtype)


def make_case(cfg: synth.Config, ln_random: bool = True, ids=None) -> Case:
    g, b = synth.ln_params(cfg, random=ln_random)
    return Case(cfg, synth.offsets(cfg), synth.token_ids(cfg) if ids is None else ids,
                synth.hidden(cfg, n=None if ids is None else len(ids)),
                synth.table(cfg, "W_K"), synth.table(cfg, "W_V"), synth.dense(cfg, "W_up"),
                synth.dense(cfg, "W_mix"), g, b)


def rowwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.max(np.abs(got - ref), axis=1)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(num / den)) if len(ref) else 0.0


def dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_np(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


class Gpu:
    """A case uploaded once, with a plan."""

    def __init__(self, case: Case):
        import torch
        import static_token_routed_amd as l3
        c, dt = case, case.cfg.dtype
        self.case = case
        self.x, self.WK, self.WV = dev(c.x, dt), dev(c.WK, dt), dev(c.WV, dt)
        self.Wup, self.Wmix = dev(c.Wup, dt), dev(c.Wmix, dt)
        self.gamma = torch.from_numpy(c.gamma).cuda()
        self.beta = torch.from_numpy(c.beta).cuda()
        self.ids = torch.from_numpy(np.ascontiguousarray(c.ids, dtype=np.int32)).cuda()
        cfg = c.cfg
        self.plan = l3.L3Plan(c.off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, dt, cfg.ln_eps)

    def forward(self, x=None, ids=None, Wmix=None, Wup=None):
        return self.plan.forward(self.x if x is None else x, self.ids if ids is None else ids,
                                 self.WK, self.WV, self.Wup if Wup is None else Wup, self.gamma,
                                 self.beta, self.Wmix if Wmix is None else Wmix)

    def close(self):
        self.plan.close()


def oracle_out(case: Case, rows=None, Wmix=None, Wup=None, stages=False, x=None):
    """fp64 oracle output for all tokens, or for the batch positions in ``rows``
    (the tables are cut down to the rows of the sampled IDs, offsets rebuilt)."""
    c = case
    f = c.f32
    Wmix = f(c.Wmix) if Wmix is None else Wmix
    Wup = f(c.Wup) if Wup is None else Wup
    x = c.x if x is None else x
    if rows is None:
        return oracle.forward(c.off, c.cfg.k, f(x), c.ids, f(c.WK), f(c.WV), Wup, c.gamma, c.beta,
                              Wmix, eps=c.cfg.ln_eps, stages=stages)
    rows = np.asarray(rows)
    ids = c.ids[rows]
    u, inv = np.unique(ids, return_inverse=True)
    d = c.off[u + 1] - c.off[u]
    off = np.concatenate([[0], np.cumsum(d)]).astype(np.int64)
    sel = np.concatenate([np.arange(c.off[t], c.off[t + 1]) for t in u])
    return oracle.forward(off, c.cfg.k, f(x[rows]), inv.astype(np.int32), f(c.WK[sel]),
                          f(c.WV[sel]), Wup, c.gamma, c.beta, Wmix, eps=c.cfg.ln_eps, stages=stages)


def sample_rows(ids: np.ndarray, n_pick: int = 96, seed: int = 0) -> np.ndarray:
    """Batch positions covering the largest blocks, single-token blocks, the first
    and last positions, and random ones."""
    rng = np.random.default_rng(seed)
    u, inv, cnt = np.unique(ids, return_inverse=True, return_counts=True)
    big = np.argsort(-cnt)[:8]
    pick = [np.flatnonzero(inv == b)[:3] for b in big]
    singles = np.flatnonzero(cnt[inv] == 1)
    pick.append(singles[:16])
    pick.append(np.array([0, len(ids) - 1]))
    pick.append(rng.choice(len(ids), size=n_pick, replace=False))
    return np.unique(np.concatenate(pick))
