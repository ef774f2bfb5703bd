"""GPU parity of the backward pass (l3_backward through the C ABI) against the
fp64 oracle's gradients on the same inputs.

Per gradient row (rows of dx, dW_K, dW_V, dW_up, dW_mix; dgamma and dbeta are
one row each): ||g_i - r_i||_inf / ||r_i||_inf <= 1e-5 (fp32 plans) or 1e-2 (bf16 plans),
key / value rows with the rounding allowance of table_row_check where their
products cancel (bf16 plans: the dense products take bf16 operands -- dout, [y ; x], dh, o --
with fp32 accumulation, and o, h, y, dh are stored in bf16).  Also: bit-for-bit
reproducibility, the accumulate-into semantics of the parameter gradients, and
rows of IDs absent from the batch left untouched."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import dev, make_case, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
l3 = pytest.importorskip("static_token_routed_amd")

CASES = {
    # fp32, dims not multiples of 64
    "f32_ragged": synth.small("bf32", vocab=300, k=24, d_in=96, d_emb=48, d_up=80, d_out=72, n=333,
                              v=2400, dtype="f32", seed=7),
    # bf16, 200 tokens: W_up recomputed by the small-batch GEMM
    "bf16_n200": synth.small("bb1", vocab=400, k=40, d_in=256, d_emb=128, d_up=256, d_out=192,
                             n=200, v=4000, dtype="bf16", seed=8, ids_s=1.05),
    # bf16, 1100 tokens (ragged against every tile): the 256x256 GEMM
    "bf16_n1100": synth.small("bb2", vocab=600, k=64, d_in=512, d_emb=256, d_up=512, d_out=256,
                              n=1100, v=9000, dtype="bf16", seed=9, ids_s=1.05),
    # bf16, the paper's d_in and d_emb (matrix-core attention backward, 8 wavefronts)
    "bf16_d2048": synth.small("bb3", vocab=300, k=96, d_in=2048, d_emb=512, d_up=512, d_out=256,
                              n=700, v=6000, dtype="bf16", seed=10, ids_s=1.05),
    # bf16, d_in 1024 / d_emb 128 (matrix-core attention backward, 4 wavefronts), blocks
    # longer than 16 tokens and 16 rows, and a ragged last row chunk (k = 70)
    "bf16_d1024_e128": synth.small("bb4", vocab=150, k=70, d_in=1024, d_emb=128, d_up=256,
                                   d_out=128, n=900, v=4000, dtype="bf16", seed=11, ids_s=1.05),
    # bf16, 4200 tokens: the parameter-gradient GEMMs (K = tokens, few output tiles)
    # split K into fp32 slabs added in order
    "bf16_n4200_splitk": synth.small("bb5", vocab=500, k=16, d_in=1024, d_emb=128, d_up=256,
                                     d_out=128, n=4200, v=3000, dtype="bf16", seed=12, ids_s=1.05),
}
KEYS = ["dx", "dW_K", "dW_V", "dW_up", "dgamma", "dbeta", "dW_mix"]


def _dout(case):
    cfg = case.cfg
    rng = np.random.default_rng(cfg.seed + 100)
    dout32 = rng.standard_normal((cfg.n, cfg.d_out)).astype(np.float32)
    return synth.f32_to_bf16_bits(dout32) if cfg.dtype == "bf16" else dout32


def _run(case, fill=0.0, reps=1, x=None, ids=None, dout=None, status=None):
    """l3_backward on the case (or on x / ids / dout given for a changed batch)."""
    cfg = case.cfg
    dt = cfg.dtype
    x = case.x if x is None else x
    ids = case.ids if ids is None else ids
    dout = _dout(case) if dout is None else dout
    n = len(ids)
    plan = l3.L3Plan(case.off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, dt, cfg.ln_eps)
    v = int(case.off[-1])
    z = lambda *shape: torch.full(shape, fill, dtype=torch.float32, device="cuda")
    g = {"dx": z(n, cfg.d_in), "dW_K": z(v, cfg.d_in), "dW_V": z(v, cfg.d_emb),
         "dW_up": z(cfg.d_up, cfg.d_emb), "dgamma": z(cfg.d_up), "dbeta": z(cfg.d_up),
         "dW_mix": z(cfg.d_out, cfg.d_up + cfg.d_in)}
    ws = torch.empty(l3.l3_backward_workspace_size(plan.handle, n), dtype=torch.uint8, device="cuda")
    args = [dev(x, dt), torch.from_numpy(np.ascontiguousarray(ids)).cuda(), n, dev(case.WK, dt),
            dev(case.WV, dt), dev(case.Wup, dt), torch.from_numpy(case.gamma).cuda(),
            torch.from_numpy(case.beta).cuda(), dev(case.Wmix, dt), dev(dout, dt)]
    for _ in range(reps):
        l3.l3_backward(plan.handle, *args, *[g[k] for k in KEYS], ws, ws.numel())
    torch.cuda.synchronize()
    # the route's flag sits at the start of the backward workspace
    assert l3.l3_status(ws) == (l3.L3_OK if status is None else status)
    plan.close()
    return {k: to_np(t) for k, t in g.items()}, synth.as_f32(dout, dt)


def _ref(case, dout):
    f = case.f32
    return oracle.backward(case.off, case.cfg.k, f(case.x), case.ids, f(case.WK), f(case.WV),
                           f(case.Wup), case.gamma, case.beta, f(case.Wmix), dout, eps=case.cfg.ln_eps,
                           magnitudes=True)


FLOOR = 1e-3  # dx, dW_up, dW_mix rows below this fraction of the tensor's max: absolute error
MAG_FACTOR = 4.0  # rounding-error allowance, in units of u * (size of the products)


def rowwise_err_floor(got: np.ndarray, ref: np.ndarray) -> tuple[float, int]:
    """max over rows of ||g_i - r_i||_inf / max(||r_i||_inf, FLOOR * ||r||_inf), and how
    many rows fall under the floor.  Each row is judged against its own size, so a
    small row cannot hide behind the tensor's largest one.  A vector is one row."""
    g2 = got.reshape(len(got), -1) if got.ndim > 1 else got.reshape(1, -1)
    r2 = ref.reshape(len(ref), -1) if ref.ndim > 1 else ref.reshape(1, -1)
    top = float(np.max(np.abs(r2))) if r2.size else 0.0
    rn = np.max(np.abs(r2), axis=1)
    den = np.maximum(rn, max(FLOOR * top, 1e-30))
    err = np.max(np.abs(g2 - r2), axis=1) / den
    return (float(err.max()) if len(err) else 0.0), int(np.sum(rn < FLOOR * top))


def table_row_check(got, ref, mag, tol, u):
    """Key / value gradient rows: ||g_j - r_j||_inf <= max(tol ||r_j||_inf, 4 u mag_j).

    A key row's gradient sum_i dS_ij x_i takes dS_ij = p_ij (<V_j, do_i> - <o_i, do_i>),
    the difference of two inner products.  Where they nearly cancel, the row is far
    smaller than the products it is formed from, and rounding do and o to the operand
    precision (unit roundoff u) moves it by about u times their size (mag_j, the
    oracle's kmag), which can be many times the row itself.  So each row is held to
    the tolerance of its own norm or to 4 u mag_j, whichever is larger; rows without
    such cancellation (4 u mag_j <= tol ||r_j||) are held to tol of their own norm.
    Returns (worst ratio to the allowance, rows under the magnitude allowance, worst
    relative error among the other rows, max ||g_j - r_j|| / (u mag_j))."""
    rn = np.max(np.abs(ref), axis=1)
    e = np.max(np.abs(got - ref), axis=1)
    allow = np.maximum(tol * rn, MAG_FACTOR * u * mag)
    allow = np.maximum(allow, 1e-300)
    plain = MAG_FACTOR * u * mag <= tol * rn
    rel_plain = float(np.max(e[plain] / np.maximum(rn[plain], 1e-300))) if plain.any() else 0.0
    units = float(np.max(e / np.maximum(u * mag, 1e-300)))
    return float(np.max(e / allow)), int(np.sum(~plain)), rel_plain, units


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    """dx, dW_up, dW_mix: every row within the tolerance of its own norm.  dW_K, dW_V:
    every touched row within the tolerance of its own norm or the rounding allowance of
    the products it is formed from (table_row_check); untouched rows exactly zero.
    dgamma, dbeta (one vector each): normwise within the tolerance."""
    print(f"backward case {name}", flush=True)
    case = make_case(CASES[name])
    got, dout = _run(case)
    ref = _ref(case, dout)
    bf16 = case.cfg.dtype == "bf16"
    tol = 1e-2 if bf16 else 1e-5
    # unit roundoff of the operands the attention gradients are formed from: bf16
    # (do, o, dS rounded to bf16), or fp32 sums over d_emb products
    u = 2.0 ** -9 if bf16 else np.sqrt(case.cfg.d_emb) * 2.0 ** -24
    touched = np.zeros(int(case.off[-1]), bool)
    for t in np.unique(case.ids):
        touched[case.off[t]:case.off[t + 1]] = True
    for k in KEYS:
        g, r = got[k], ref[k]
        if k in ("dW_K", "dW_V"):
            assert np.all(g[~touched] == 0.0), f"{k}: rows of absent IDs changed"
            mag = ref["kmag" if k == "dW_K" else "vmag"][touched]
            ratio, n_mag, rel, units = table_row_check(g[touched], r[touched], mag, tol, u)
            print(f"  {k}: worst row at {ratio:.2f} of its allowance over {int(touched.sum())} rows "
                  f"({n_mag} under the rounding allowance); other rows max rel err {rel:.2e}; "
                  f"max error {units:.2f} u * mag", flush=True)
            assert ratio <= 1.0, f"{name} {k}: a row at {ratio:.2f} of its allowance"
            assert rel <= tol
            continue
        err, small = rowwise_err_floor(g, r)
        print(f"  {k}: worst row err {err:.2e} over {len(r)} rows ({small} under the floor)",
              flush=True)
        assert err <= tol, f"{name} {k}: {err:.3e} > {tol}"


@pytest.mark.parametrize("name", ["bf16_n200", "bf16_n4200_splitk"])
def test_backward_deterministic_and_accumulates(name):
    case = make_case(CASES[name])
    a, _ = _run(case)
    b, _ = _run(case)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), f"{k} not reproducible"
    # two calls into the same buffers: parameter gradients doubled exactly, dx written
    c, _ = _run(case, reps=2)
    for k in KEYS:
        want = a[k] if k == "dx" else 2.0 * a[k]
        assert np.array_equal(c[k], want), k


def test_backward_untouched_rows():
    case = make_case(CASES["bf16_n200"])
    got, _ = _run(case, fill=7.0)
    touched = np.zeros(int(case.off[-1]), bool)
    for t in np.unique(case.ids):
        touched[case.off[t]:case.off[t + 1]] = True
    for k in ("dW_K", "dW_V"):
        assert np.all(got[k][~touched] == 7.0), f"{k}: rows of absent IDs changed"


def test_backward_out_of_range_ids():
    # IDs outside [0, vocab) are flagged and add no attention gradient.  They sort
    # after every valid ID, so every other token keeps its sorted place: the key /
    # value gradients and the other tokens' dx equal, bit for bit, those of the batch
    # without those tokens (matrix-core kernels: d_in 1024, d_emb 128).
    case = make_case(CASES["bf16_d1024_e128"])
    cfg = case.cfg
    dout = _dout(case)
    bad = [5, 300, 301]
    ids = case.ids.copy()
    ids[5], ids[300], ids[301] = -3, cfg.vocab, cfg.vocab + 7
    got, _ = _run(case, ids=ids, dout=dout, status=l3.L3_ERR_TOKEN_RANGE)
    keep = np.ones(cfg.n, bool)
    keep[bad] = False
    ref, _ = _run(case, x=case.x[keep], ids=case.ids[keep], dout=dout[keep])
    for k in KEYS:
        assert np.all(np.isfinite(got[k])), k
    assert np.array_equal(got["dW_K"], ref["dW_K"])
    assert np.array_equal(got["dW_V"], ref["dW_V"])
    assert np.array_equal(got["dx"][keep], ref["dx"])
