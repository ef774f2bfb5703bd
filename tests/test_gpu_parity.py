"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Route outputs must match bit for bit; float outputs within the row-normwise
tolerance (1e-5 fp32, 2e-2 bf16) of gpu_cases.py."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_cases import Case, Gpu, dev, make_case, oracle_out, rowwise_err, sample_rows, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
l3 = pytest.importorskip("static_token_routed_amd")


def _route_case(name):
    rng = np.random.default_rng(ROUTE_CASES.index(name))
    if name in ("tiny_f32", "small_bf16", "paper_bf16", "skew_bf16"):
        cfg = synth.CONFIGS[name]
        return synth.offsets(cfg), synth.token_ids(cfg)
    vocab = 180000
    off = np.arange(vocab + 1, dtype=np.int64)  # d_t = 1 everywhere
    if name == "all_equal":
        ids = np.full(5000, 77, np.int32)
    elif name == "all_distinct":
        ids = rng.permutation(6000).astype(np.int32)
    elif name == "single":
        ids = np.array([vocab - 1], np.int32)
    elif name == "ragged":
        ids = rng.integers(0, 50, size=3 * 2048 + 1).astype(np.int32)
    elif name == "max_id":
        ids = np.where(rng.random(4099) < 0.5, vocab - 1, 0).astype(np.int32)
    elif name == "out_of_range":
        ids = rng.integers(-3, vocab + 3, size=2500).astype(np.int32)
        ids[:6] = [-1, vocab, vocab + 100, 2 ** 31 - 1, -(2 ** 31), 5]
    # batches of at most 1024 tokens take the one-workgroup route
    elif name == "small_zipf":
        ids = synth.token_ids(synth.CONFIGS["paper_bf16"])[:1000].copy()
    elif name == "small_out_of_range":
        ids = rng.integers(-2, 40, size=700).astype(np.int32)
        ids[:4] = [vocab, -(2 ** 31), 2 ** 31 - 1, vocab + 7]
    elif name in ("n1024", "n1025"):
        ids = rng.integers(0, 300, size=int(name[1:])).astype(np.int32)
    # more than 64 tiles of 512 keys: the scatter offsets come from one pass over the
    # histogram first
    elif name == "tiles_2048":
        ids = rng.integers(0, vocab, size=1 << 20).astype(np.int32)
    elif name == "tiles_65":
        ids = rng.integers(0, 700, size=64 * 512 + 1).astype(np.int32)
    # the last batch whose scatter reads the whole histogram (16 tiles) and the first that
    # takes the digit scan (17)
    elif name in ("tiles_16", "tiles_17"):
        n = 16 * 512 + (name == "tiles_17")
        ids = rng.integers(0, 900, size=n).astype(np.int32)
    else:
        raise KeyError(name)
    return off, ids


ROUTE_CASES = ["tiny_f32", "small_bf16", "paper_bf16", "skew_bf16", "all_equal", "all_distinct",
               "single", "ragged", "max_id", "out_of_range", "small_zipf", "small_out_of_range",
               "n1024", "n1025", "tiles_16", "tiles_17", "tiles_65", "tiles_2048"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_bit_exact(name):
    off, ids = _route_case(name)
    vocab = len(off) - 1
    print(f"route case {name}: n={len(ids)} vocab={vocab}", flush=True)
    plan = l3.L3Plan(off, int(np.max(np.diff(off))), 64, 64, 64, 64, "bf16")
    r = plan.route(torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    ref = oracle.route(ids, vocab)
    m = int(r["num_segments"].item())
    assert m == ref["num_segments"]
    for key in ("perm", "sorted_ids", "inv_perm"):
        assert np.array_equal(to_np(r[key]), ref[key]), key
    for key in ("uniq", "counts"):
        assert np.array_equal(to_np(r[key])[:m], ref[key]), key
    assert np.array_equal(to_np(r["seg_start"])[:m + 1], ref["seg_start"])
    status = plan.status()
    assert status == (l3.L3_ERR_TOKEN_RANGE if ref["err"] else l3.L3_OK)
    plan.close()


def test_tiny_f32_full():
    case = make_case(synth.CONFIGS["tiny_f32"])
    g = Gpu(case)
    got = to_np(g.forward())
    err = rowwise_err(got, oracle_out(case))
    print(f"tiny_f32 err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


SMALL_BF16 = [
    # name, vocab, k, d_in, d_emb, d_up, d_out, n, v
    ("d64", 200, 16, 64, 64, 64, 64, 300, 1200),
    ("d512_e128", 500, 40, 512, 128, 256, 192, 1000, 6000),
    ("d1024_e256", 800, 64, 1024, 256, 512, 320, 2600, 20000),
    ("d2048_e512", 600, 96, 2048, 512, 512, 256, 1500, 20000),
    ("d4096_e512", 400, 64, 4096, 512, 256, 256, 700, 9000),
    # d_in 4096 with d_emb 256: the streaming items' quarter layout with one V stage
    ("d4096_e256", 300, 80, 4096, 256, 256, 256, 900, 9000),
    ("ragged_e64", 50, 200, 192, 64, 128, 64, 513, 3000),
    # MFMA path over several 128-row softmax groups, a partial last group, and
    # blocks longer than 512 rows, for each V stage shape (d_emb 64 / 256 / 512)
    ("groups_d128_e64", 80, 300, 128, 64, 128, 128, 800, 8000),
    ("groups_d256_e256_k700", 60, 700, 256, 256, 256, 128, 600, 12000),
    ("groups_d1024_e512", 100, 260, 1024, 512, 256, 256, 700, 9000),
    # small batches (split-K GEMMs, LayerNorm applied while staging h), random
    # gamma / beta: a ragged 64-row tile, a W_mix K split that straddles the h|x
    # seam (d_up 320), and the largest batch of that path
    ("skinny_d1024_e256", 800, 64, 1024, 256, 512, 320, 200, 20000),
    ("skinny_straddle", 300, 48, 1024, 128, 320, 192, 77, 8000),
    ("skinny_d2048_e512_n512", 600, 96, 2048, 512, 512, 256, 512, 20000),
    # batches of at most 512 tokens take the split-row gather: d_in below one
    # 512-column slice (masked lanes, 16-row chunks) at the largest such batch, the
    # widest d_in (2-row chunks, one token per group), and one token past the limit
    # (the single-workgroup route with the per-block gather kernels)
    # 17 route tiles: the digit-scan scatter, then the factored W_mix
    ("d1024_n8193", 2000, 96, 1024, 256, 256, 256, 8193, 40000),
    ("split_d192_n512", 300, 90, 192, 64, 128, 64, 512, 9000),
    ("split_d4096_e128", 200, 40, 4096, 128, 128, 128, 100, 4000),
    ("nosplit_d192_n513", 300, 90, 192, 64, 128, 64, 513, 9000),
]


@pytest.mark.parametrize("spec", SMALL_BF16, ids=[s[0] for s in SMALL_BF16])
def test_small_bf16_full(spec):
    name, vocab, k, d_in, d_emb, d_up, d_out, n, v = spec
    cfg = synth.small(name, vocab=vocab, k=k, d_in=d_in, d_emb=d_emb, d_up=d_up, d_out=d_out, n=n,
                      v=v, dtype="bf16", ids_s=1.05)
    print(f"bf16 case {name}", flush=True)
    case = make_case(cfg, ln_random=name.startswith("skinny"))
    g = Gpu(case)
    got = to_np(g.forward())
    err = rowwise_err(got, oracle_out(case))
    print(f"bf16 case {name}: err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


@pytest.mark.parametrize("n", [900, 200])
def test_stage_identities(n):
    """W_mix = [0 | I] returns x exactly; W_mix = [I | 0] returns LN(h) (oracle's y)."""
    cfg = synth.small("ident", vocab=300, k=32, d_in=256, d_emb=128, d_up=256, d_out=256, n=n,
                      v=3000, dtype="bf16")
    case = make_case(cfg)
    g = Gpu(case)
    I, Z = np.eye(256, dtype=np.float32), np.zeros((256, 256), np.float32)
    w0 = synth.f32_to_bf16_bits(np.concatenate([Z, I], 1))
    got = g.forward(Wmix=dev(w0, "bf16"))
    assert torch.equal(got, g.x), "W_mix = [0 | I] must reproduce x bit for bit"
    w1 = np.concatenate([I, Z], 1)
    got = to_np(g.forward(Wmix=dev(synth.f32_to_bf16_bits(w1), "bf16")))
    _, o, h, y = oracle_out(case, stages=True)
    err = rowwise_err(got, y)
    print(f"LN(h) stage err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


def test_gemm_bf16_standalone():
    rng = np.random.default_rng(5)
    for M, N, K in [(64, 8192, 2048), (300, 320, 192), (1, 64, 64), (513, 1024, 4096),
                    (65, 1024, 320), (512, 192, 2112), (16, 64, 4096)]:
        a = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        b = synth.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K))
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        l3.l3_gemm_bf16(dev(a, "bf16"), dev(b, "bf16"), C, M, N, K)
        ref = synth.bf16_bits_to_f32(a).astype(np.float64) @ synth.bf16_bits_to_f32(b).astype(np.float64).T
        err = rowwise_err(to_np(C), ref)
        print(f"gemm {M}x{N}x{K}: err {err:.2e}", flush=True)
        assert err <= 8e-3


@pytest.fixture(scope="module")
def small_cfg_gpu():
    case = make_case(synth.CONFIGS["small_bf16"])
    g = Gpu(case)
    yield g
    g.close()


def test_small_bf16_config_full(small_cfg_gpu):
    """Every one of the small bf16 workload's 16384 output rows against the oracle."""
    g = small_cfg_gpu
    case = g.case
    got = to_np(g.forward())
    assert np.all(np.isfinite(got))
    errs = []
    for c0 in range(0, len(case.ids), 8192):
        r = np.arange(c0, min(c0 + 8192, len(case.ids)))
        errs.append(rowwise_err(got[r], oracle_out(case, rows=r)))
    err = max(errs)
    print(f"small_bf16 config: all {len(case.ids)} tokens, max row-normwise err {err:.2e}", flush=True)
    assert err <= case.tol


def _close(a, b, tol):
    err = rowwise_err(to_np(a), to_np(b))
    assert err <= tol, f"rel err {err:.2e}"
    return err


def test_determinism_and_batch_independence(small_cfg_gpu):
    """Bitwise run-to-run determinism.  A sub-batch, or a shuffled batch, gives the
    same rows within the parity tolerance (a token may be computed in a different
    work-item grouping, so bit equality is not promised across batches)."""
    g = small_cfg_gpu
    a = g.forward().clone()
    b = g.forward()
    assert torch.equal(a, b), "two runs differ"
    sel = torch.arange(0, g.ids.numel(), 7, device="cuda")
    sub = g.forward(x=g.x[sel].contiguous(), ids=g.ids[sel].contiguous())
    e1 = _close(sub, a[sel], g.case.tol)
    p = torch.randperm(g.ids.numel(), device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    sh = g.forward(x=g.x[p].contiguous(), ids=g.ids[p].contiguous())
    e2 = _close(sh, a[p], g.case.tol)
    print(f"sub-batch err {e1:.2e}, shuffled err {e2:.2e}", flush=True)


def test_out_of_range_ids_small_batch(small_cfg_gpu):
    # 300 tokens take the small-batch route and the split-row gather
    g = small_cfg_gpu
    x, ids = g.x[:300].contiguous(), g.ids[:300].clone()
    ids[7] = -5
    ids[250] = g.case.cfg.vocab + 1
    out = g.forward(x=x, ids=ids)
    assert g.plan.status() == l3.L3_ERR_TOKEN_RANGE
    good = g.forward(x=x, ids=g.ids[:300].contiguous())
    assert g.plan.status() == l3.L3_OK
    keep = torch.ones(300, dtype=torch.bool, device="cuda")
    keep[7] = keep[250] = False
    assert torch.equal(out[keep], good[keep])
    assert torch.isfinite(out.float()).all()


def test_out_of_range_ids_flag(small_cfg_gpu):
    g = small_cfg_gpu
    ids = g.ids.clone()
    ids[5] = -1
    ids[100] = g.case.cfg.vocab
    out = g.forward(ids=ids)
    assert g.plan.status() == l3.L3_ERR_TOKEN_RANGE
    good = g.forward()
    assert g.plan.status() == l3.L3_OK
    keep = torch.ones(ids.numel(), dtype=torch.bool, device="cuda")
    keep[5] = keep[100] = False
    _close(out[keep], good[keep], g.case.tol)
    assert torch.isfinite(out.float()).all()


def test_zero_and_one_token(small_cfg_gpu):
    g = small_cfg_gpu
    out = torch.empty((0, g.case.cfg.d_out), dtype=torch.bfloat16, device="cuda")
    ws = g.plan.workspace(1)
    l3.l3_forward(g.plan.handle, g.x, g.ids, 0, g.WK, g.WV, g.Wup, g.gamma, g.beta, g.Wmix, out,
                  ws, ws.numel())
    one = g.forward(x=g.x[3:4].contiguous(), ids=g.ids[3:4].contiguous())
    ref = oracle_out(g.case, rows=[3])
    assert rowwise_err(to_np(one), ref) <= g.case.tol


def test_workspace_too_small(small_cfg_gpu):
    g = small_cfg_gpu
    n = g.ids.numel()
    out = torch.empty((n, g.case.cfg.d_out), dtype=torch.bfloat16, device="cuda")
    need = l3.l3_workspace_size(g.plan.handle, n)
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(l3.L3Error) as e:
        l3.l3_forward(g.plan.handle, g.x, g.ids, n, g.WK, g.WV, g.Wup, g.gamma, g.beta, g.Wmix,
                      out, ws, ws.numel())
    assert e.value.code == l3.L3_ERR_CAPACITY


DECODE_CASES = {
    "decode_bf16": synth.CONFIGS["decode_bf16"],
    # rows of 320 16-byte chunks: two rounds of the staging copy, K/V seam inside one
    "wide_bf16": dataclasses.replace(
        synth.small("wide", vocab=5000, k=256, d_in=2048, d_emb=512, d_up=512, d_out=512,
                    n=64, v=60000, dtype="bf16", seed=3), ids_s=1.05),
    "decode_f32": synth.small("dec32", vocab=3000, k=96, d_in=256, d_emb=128, d_up=256,
                              d_out=256, n=64, v=40000, dtype="f32", seed=4),
    # fp32 rows that are not whole 16-byte chunks (400 and 148 bytes): the staging copy
    # moves them in 4-byte elements
    "decode_f32_odd": synth.small("dec32o", vocab=3000, k=96, d_in=100, d_emb=37, d_up=72,
                                  d_out=52, n=64, v=40000, dtype="f32", seed=5),
}


def _pinned(a, dtype):
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(a)
    return t.pin_memory()


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_staged_equals_resident(name):
    """Pinned-host tables + prefetch of the step's rows + staged forward give the
    same bits as the forward over device-resident tables."""
    cfg = DECODE_CASES[name]
    print(f"decode case {name}", flush=True)
    case = make_case(cfg, ln_random=True)
    g = Gpu(case)
    WKh, WVh = _pinned(case.WK, cfg.dtype), _pinned(case.WV, cfg.dtype)
    st = l3.l3_staging_create(g.plan.handle, 64 * cfg.k, 64)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ws = g.plan.workspace(64)
    for step in range(5):
        n = (64, 64, 1, 37, 64)[step]
        if step == 0:  # the case's own batch, also checked against the oracle
            ids, x = np.ascontiguousarray(case.ids, dtype=np.int32), g.x
        else:
            ids = synth.token_ids(cfg, n=n, step=step)
            x = dev(synth.hidden(cfg, n=n, step=step), cfg.dtype)
        l3.l3_prefetch(g.plan.handle, ids, n, WKh, WVh, st, side, ev)
        torch.cuda.current_stream().wait_event(ev)
        out = torch.empty((n, cfg.d_out), dtype=x.dtype, device="cuda")
        l3.l3_forward_staged(st, x, n, g.Wup, g.gamma, g.beta, g.Wmix, out, ws, ws.numel())
        ref = g.forward(x=x, ids=torch.from_numpy(ids).cuda())
        assert torch.equal(out, ref), f"step {step}"
        if step == 0:
            err = rowwise_err(to_np(out), oracle_out(case))
            print(f"decode {name} staged vs oracle err {err:.2e}", flush=True)
            assert err <= case.tol
    torch.cuda.synchronize()
    with pytest.raises(l3.L3Error) as e:
        l3.l3_prefetch(g.plan.handle, np.array([cfg.vocab], np.int32), 1, WKh, WVh, st, side, ev)
    assert e.value.code == l3.L3_ERR_TOKEN_RANGE
    # a device cache of the hot IDs' rows: same bits, fewer rows over PCIe
    hot = np.argsort(-np.bincount(case.ids, minlength=cfg.vocab))[:40].astype(np.int32)
    l3.l3_staging_set_cache(st, hot, WKh, WVh)
    for step in (0, 5):
        n = 64
        ids = np.ascontiguousarray(case.ids, dtype=np.int32) if step == 0 else synth.token_ids(cfg, n=n, step=step)
        x = g.x if step == 0 else dev(synth.hidden(cfg, n=n, step=step), cfg.dtype)
        l3.l3_prefetch(g.plan.handle, ids, n, WKh, WVh, st, side, ev)
        torch.cuda.current_stream().wait_event(ev)
        out = torch.empty((n, cfg.d_out), dtype=x.dtype, device="cuda")
        l3.l3_forward_staged(st, x, n, g.Wup, g.gamma, g.beta, g.Wmix, out, ws, ws.numel())
        ref = g.forward(x=x, ids=torch.from_numpy(ids).cuda())
        assert torch.equal(out, ref), f"cached step {step}"
        rows, cached = l3.l3_staging_stats(st)
        assert 0 < cached <= rows, (rows, cached)
    l3.l3_staging_set_cache(st, np.zeros(0, np.int32), WKh, WVh)
    # tables in pageable host memory have no device mapping: refused, nothing enqueued
    pageable = torch.from_numpy(np.ascontiguousarray(case.WK[:16]))
    with pytest.raises(l3.L3Error) as e:
        l3.l3_prefetch(g.plan.handle, np.array([0], np.int32), 1, pageable, WVh, st, side, ev)
    assert e.value.code == l3.L3_ERR_INVALID_ARG
    l3.l3_staging_destroy(st)
    g.close()


def full_size_rows(name: str, ids: np.ndarray) -> np.ndarray:
    """The tokens the full-size tests compare: every token of the benchmark workload;
    for the 131072-token skew pair, one token of each of the 200 forced IDs (the
    blocks at the k = 512 cap, or d_t 4 in the uniform allocation), the sampler's
    largest and single-token blocks, and seeded random tokens, 4096 or more."""
    if name == "paper_bf16":
        return np.arange(len(ids))
    first = np.array([np.flatnonzero(ids == t)[0] for t in range(200)])
    rng = np.random.default_rng(17)
    pick = np.concatenate([first, sample_rows(ids, 160), rng.choice(len(ids), 4096, replace=False)])
    return np.unique(pick)


@pytest.mark.parametrize("name", ["paper_bf16", "skew_bf16", "skew_uniform_bf16"])
def test_full_size(name):
    """Full-size workloads in the launch configuration the benchmark times: all 32768
    tokens of paper_bf16, and >= 4096 tokens of the skew stress pair (131072 tokens,
    d_in 4096, half of them on the 200 IDs at the k = 512 cap, with a Zipf-shaped or
    a uniform allocation) covering every one of the 200 forced IDs."""
    cfg = synth.CONFIGS[name]
    print(f"generating {name}", flush=True)
    case = make_case(cfg)
    g = Gpu(case)
    got = to_np(g.forward())
    assert np.all(np.isfinite(got))
    rows = full_size_rows(name, case.ids)
    if name != "paper_bf16":
        assert set(range(200)) <= set(case.ids[rows].tolist())
    errs = []
    for c0 in range(0, len(rows), 8192):  # the oracle on token chunks, tables cut to their rows
        r = rows[c0:c0 + 8192]
        errs.append(rowwise_err(got[r], oracle_out(case, rows=r)))
        print(f"{name}: tokens {c0}..{c0 + len(r)} of {len(rows)}, err {errs[-1]:.2e}", flush=True)
    err = max(errs)
    print(f"{name}: {len(rows)} tokens compared, max row-normwise err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


@pytest.mark.parametrize("d,n", [(256, 300), (256, 1200), (512, 1500), (64, 900),
                                 (1024, 1300), (1024, 300), (2048, 700), (2048, 200)])
def test_tied_tables(d, n):
    """W_V = W_K (one device table passed for both; d_emb = d_in): the forward equals
    the oracle's with equal tables (the pages' tied variant).  The wavefront kernel's
    items read each row once for both roles; at d 1024 and 2048 (the tied-only widths)
    that kernel takes every block, above 512 tokens with the factored W_mix and at or
    below with the small-batch GEMMs."""
    cfg = dataclasses.replace(
        synth.small("tied", vocab=500, k=48, d_in=d, d_emb=d, d_up=256, d_out=192, n=n,
                    v=6000, dtype="bf16", seed=11), ids_s=1.05, tied=True)
    case = make_case(cfg)
    assert np.array_equal(case.WK, case.WV)
    g = Gpu(case)
    got = to_np(g.plan.forward(g.x, g.ids, g.WK, g.WK, g.Wup, g.gamma, g.beta, g.Wmix))
    err = rowwise_err(got, oracle_out(case))
    print(f"tied d={d} n={n}: err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


def test_tied_only_widths_refuse_separate_tables():
    """bf16 plans with d_emb = d_in = 1024 serve tied tables only: a forward with a
    separate W_V, a decode staging and the backward are refused with UNSUPPORTED
    before anything is enqueued."""
    cfg = dataclasses.replace(
        synth.small("tied_only", vocab=200, k=16, d_in=1024, d_emb=1024, d_up=128, d_out=128,
                    n=600, v=2000, dtype="bf16", seed=5), ids_s=1.05, tied=True)
    case = make_case(cfg)
    g = Gpu(case)
    WV = g.WK.clone()
    with pytest.raises(l3.L3Error) as e:
        g.plan.forward(g.x, g.ids, g.WK, WV, g.Wup, g.gamma, g.beta, g.Wmix)
    assert e.value.code == l3.L3_ERR_UNSUPPORTED
    with pytest.raises(l3.L3Error) as e:
        l3.l3_staging_create(g.plan.handle, 1024, 64)
    assert e.value.code == l3.L3_ERR_UNSUPPORTED
    n = len(case.ids)
    f32 = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(l3.l3_backward_workspace_size(g.plan.handle, n), 256), dtype=torch.uint8,
                     device="cuda")
    dout = torch.zeros(n, cfg.d_out, dtype=torch.bfloat16, device="cuda")
    rc = l3._lib.l3_backward(g.plan.handle, g.x.data_ptr(), g.ids.data_ptr(), n, g.WK.data_ptr(),
                             g.WK.data_ptr(), g.Wup.data_ptr(), g.gamma.data_ptr(), g.beta.data_ptr(),
                             g.Wmix.data_ptr(), dout.data_ptr(), f32(n, cfg.d_in).data_ptr(),
                             f32(cfg.v, cfg.d_in).data_ptr(), f32(cfg.v, cfg.d_emb).data_ptr(),
                             f32(cfg.d_up, cfg.d_emb).data_ptr(), f32(cfg.d_up).data_ptr(),
                             f32(cfg.d_up).data_ptr(), f32(cfg.d_out, cfg.d_up + cfg.d_in).data_ptr(),
                             ws.data_ptr(), ws.numel(), None)
    assert rc == l3.L3_ERR_UNSUPPORTED
    # the tied forward itself runs
    got = to_np(g.plan.forward(g.x, g.ids, g.WK, g.WK, g.Wup, g.gamma, g.beta, g.Wmix))
    assert rowwise_err(got, oracle_out(case)) <= case.tol
    g.close()


@pytest.mark.parametrize("n", [900, 200])
@pytest.mark.parametrize("beta_u", [0.3, 0.5])
def test_layernorm_offset_mean(n, beta_u):
    """h with a large mean: every V row gets the same unit vector u added and every
    W_up row beta_u * u, so each token's h gains about beta_u * sqrt(d_emb) * sigma on
    all features and |mean(h)| / sigma(h) is a few units.  The LayerNorm's mean term
    then carries most of h: on batches of more than 512 tokens LayerNorm is folded
    into the W_mix weights (the mean enters as mean * (W1 gamma)), on smaller ones it
    is applied while h is staged.  Both are held to the oracle's tolerance, and the
    ratio the case reaches is printed with the error."""
    cfg = synth.small("lnmean", vocab=300, k=32, d_in=256, d_emb=128, d_up=256, d_out=256, n=n,
                      v=3000, dtype="bf16", seed=31)
    case = make_case(cfg, ln_random=True)
    u = np.full(cfg.d_emb, cfg.d_emb ** -0.5, np.float32)
    WV = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(case.WV) + u)
    Wup = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(case.Wup) + np.float32(beta_u) * u)
    case = dataclasses.replace(case, WV=WV, Wup=Wup)
    _, _, h, _ = oracle_out(case, stages=True)
    ratio = np.abs(h.mean(axis=1)) / h.std(axis=1)
    print(f"|mean(h)|/sigma(h): median {np.median(ratio):.2f}, min {ratio.min():.2f}, "
          f"max {ratio.max():.2f}", flush=True)
    assert np.median(ratio) > 1.5
    g = Gpu(case)
    got = to_np(g.forward())
    err = rowwise_err(got, oracle_out(case))
    print(f"n={n} beta_u={beta_u}: row-normwise err {err:.2e}", flush=True)
    assert err <= case.tol
    g.close()


def test_workspace_for_larger_batch_serves_smaller():
    """A workspace of l3_workspace_size(plan, 512) bytes runs every smaller batch: at the
    paper's widths with d_t up to 512, batches of about 170..256 tokens carry split-row
    partials (64 MB) that the 512-token layout does not have."""
    cfg = synth.small("wsmono", vocab=200, k=512, d_in=2048, d_emb=512, d_up=512, d_out=256,
                      n=512, v=20000, dtype="bf16", seed=33)
    case = make_case(cfg)
    assert int(np.max(np.diff(case.off))) == 512
    g = Gpu(case)
    need = l3.l3_workspace_size(g.plan.handle, 512)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for n in (200, 256, 1, 511):
        out = torch.empty((n, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        l3.l3_forward(g.plan.handle, g.x, g.ids, n, g.WK, g.WV, g.Wup, g.gamma, g.beta, g.Wmix, out,
                      ws, ws.numel())
        torch.cuda.synchronize()
        err = rowwise_err(to_np(out), oracle_out(case, rows=np.arange(n)))
        print(f"n={n} on the 512-token workspace ({need} B): err {err:.2e}", flush=True)
        assert err <= case.tol
    g.close()


def test_factored_back_to_back_weight_sets():
    """Batches of more than 512 tokens form the weight-only factors F and G on the
    plan's own stream, beside the sort and the gather.  Two forwards on one
    workspace and one non-default stream, with different W_up, gamma, beta and W_mix,
    are issued with no host synchronisation between them, twice over: the second
    call's factors must not overwrite the first call's before its W_mix GEMM has
    read them, nor run before the weights written just before the call.  Each output
    must equal, bit for bit, the same call run alone, and match the oracle."""
    cfg = synth.small("b2b", vocab=400, k=24, d_in=256, d_emb=128, d_up=512, d_out=256, n=900,
                      v=4000, dtype="bf16", seed=41)
    a = make_case(cfg, ln_random=True)
    other = make_case(dataclasses.replace(cfg, seed=cfg.seed + 7), ln_random=True)
    b = dataclasses.replace(a, Wup=other.Wup, Wmix=other.Wmix, gamma=other.gamma, beta=other.beta)
    g = Gpu(a)
    wb = {"Wup": dev(b.Wup, "bf16"), "Wmix": dev(b.Wmix, "bf16"),
          "gamma": torch.from_numpy(b.gamma).cuda(), "beta": torch.from_numpy(b.beta).cuda()}
    wa = {"Wup": g.Wup, "Wmix": g.Wmix, "gamma": g.gamma, "beta": g.beta}

    def run(w, stream=None):
        return g.plan.forward(g.x, g.ids, g.WK, g.WV, w["Wup"], w["gamma"], w["beta"], w["Wmix"],
                              stream=stream)

    alone_a = run(wa)
    torch.cuda.synchronize()
    alone_b = run(wb)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        # weights written on this stream just before the calls that read them
        wb2 = {k_: torch.empty_like(v_) for k_, v_ in wb.items()}
        for k_ in wb:
            wb2[k_].copy_(wb[k_])
        outs = [run(wa, side), run(wb2, side), run(wa, side), run(wb2, side)]
    side.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, alone_a if i % 2 == 0 else alone_b), f"call {i} differs from the call run alone"
    for case, got in ((a, alone_a), (b, alone_b)):
        err = rowwise_err(to_np(got), oracle_out(case))
        print(f"weight set {'ab'[case is b]}: err {err:.2e}", flush=True)
        assert err <= case.tol
    g.close()
