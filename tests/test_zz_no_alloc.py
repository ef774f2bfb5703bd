"""l3_forward_noalloc (the workspace in the library's own device array) against
l3_forward (a caller workspace): the same kernels, so the same bits, on two calls in
a row with the second batch smaller than the first (a large batch through the
256x256 GEMMs, then a small one through the split-row gather and split-K GEMMs,
whose stale contents from the first call must not leak), plus the oracle on the
first; and the host-side rejection of a batch whose workspace exceeds the array."""
import numpy as np
import pytest

import synth
from gpu_cases import Gpu, make_case, oracle_out, rowwise_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
l3 = pytest.importorskip("static_token_routed_amd")


def test_forward_noalloc_matches_forward():
    cfg = synth.small("noalloc", vocab=600, k=96, d_in=1024, d_emb=256, d_up=512, d_out=320,
                      n=1500, v=20000, dtype="bf16", seed=41, ids_s=1.05)
    case = make_case(cfg, ln_random=True)
    g = Gpu(case)
    for n in (1500, 200):
        print(f"noalloc call with {n} tokens", flush=True)
        x, ids = g.x[:n].contiguous(), g.ids[:n].contiguous()
        got = torch.empty((n, cfg.d_out), dtype=torch.bfloat16, device="cuda")
        l3.l3_forward_noalloc(g.plan.handle, x, ids, n, g.WK, g.WV, g.Wup, g.gamma, g.beta, g.Wmix,
                              got)
        want = g.forward(x=x, ids=ids)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"n={n}: differs from l3_forward"
        err = rowwise_err(to_np(got), oracle_out(case, rows=np.arange(n)))
        print(f"n={n}: bitwise equal to l3_forward; oracle err {err:.2e}", flush=True)
        assert err <= case.tol
    g.close()


def test_forward_noalloc_capacity():
    # d_in = d_up = d_out = 4096 with d_t up to 512: 31 tokens fit in 64 MiB, 2000 do not
    cfg = synth.small("noalloc_big", vocab=100, k=512, d_in=4096, d_emb=512, d_up=4096,
                      d_out=4096, n=2000, v=20000, dtype="bf16", seed=42)
    off = synth.offsets(cfg)
    plan = l3.L3Plan(off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, "bf16")
    assert l3.l3_workspace_size(plan.handle, 2000) > 64 << 20
    # buffers of the full sizes (never read: the call is refused on the host first)
    n = 2000
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((n, cfg.d_in), **bf)
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    WK, WV = torch.zeros((cfg.v, cfg.d_in), **bf), torch.zeros((cfg.v, cfg.d_emb), **bf)
    Wup, Wmix = torch.zeros((cfg.d_up, cfg.d_emb), **bf), torch.zeros((cfg.d_out, cfg.d_up + cfg.d_in), **bf)
    g = torch.ones(cfg.d_up, dtype=torch.float32, device="cuda")
    out = torch.empty((n, cfg.d_out), **bf)
    with pytest.raises(l3.L3Error) as e:
        l3.l3_forward_noalloc(plan.handle, x, ids, n, WK, WV, Wup, g, g, Wmix, out)
    assert e.value.code == l3.L3_ERR_CAPACITY
    plan.close()
