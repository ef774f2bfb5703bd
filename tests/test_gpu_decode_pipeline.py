"""GPU test of the two-layer decode pipeline (DecodeLayers over the C ABI).

The pages place the lookup layers after several decoder layers and prefetch each
layer's rows from host memory as soon as the token is sampled, so the copies run
under the layers before them (papernotes.org page, section 关键设计 item 3;
sciencestack.ai page, Fig. 4 caption).  Here two layers with their own tables
in pinned host memory run several decode steps with no host synchronisation
between them: at each step's start both prefetches are issued, each on its own
side stream; the main stream runs a pre-layer GEMM, layer 1, the GEMM again (the
layers in between), then layer 2 on layer 1's output.  Every layer output of
every step must equal, bit for bit, the forward over device-resident tables on
the same input; layer 1 (and layer 2, given layer 1's output) must match the
oracle.  Run without and with a device cache of the hot IDs' rows.
"""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_cases import dev, make_case, oracle_out, rowwise_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
l3 = pytest.importorskip("static_token_routed_amd")

STEP_TOKENS = (64, 64, 37, 64, 1, 64, 50, 64)


def _layer(case):
    cfg = case.cfg
    pinned = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).pin_memory()
    plan = l3.L3Plan(case.off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, "bf16", cfg.ln_eps)
    return {"plan": plan, "W_K_host": pinned(case.WK), "W_V_host": pinned(case.WV),
            "W_up": dev(case.Wup, "bf16"), "gamma": torch.from_numpy(case.gamma).cuda(),
            "beta": torch.from_numpy(case.beta).cuda(), "W_mix": dev(case.Wmix, "bf16"),
            # device-resident copies for the reference forward
            "WK": dev(case.WK, "bf16"), "WV": dev(case.WV, "bf16")}


@pytest.mark.parametrize("cached", [False, True], ids=["uncached", "hot_rows_cached"])
def test_two_layer_decode_pipeline(cached):
    base = synth.CONFIGS["decode_bf16"]
    assert base.d_out == base.d_in, "layer 2 reads layer 1's output"
    c1 = make_case(base, ln_random=True)
    c2 = make_case(dataclasses.replace(base, seed=base.seed + 1), ln_random=True)
    L = [_layer(c1), _layer(c2)]
    pipe = l3.DecodeLayers(L, max_tokens=64)
    hot = np.arange(40, dtype=np.int32)
    if cached:
        pipe.set_cache(0, hot)
        pipe.set_cache(1, hot)
    pa, pb = (dev(a, "bf16") for a in synth.pre_gemm_operands(base))
    pc = torch.empty((base.pre_m, base.pre_n), dtype=torch.bfloat16, device="cuda")

    def gemm():  # stand-in for the decoder layers before and between the lookup layers
        l3.l3_gemm_bf16(pa, pb, pc, base.pre_m, base.pre_n, base.pre_k)

    steps, served = [], 0
    for s, n in enumerate(STEP_TOKENS):
        ids = synth.token_ids(base, n=n, step=s)
        x = dev(synth.hidden(base, n=n, step=s), "bf16")
        pipe.prefetch(ids)               # both layers' copies start now
        gemm()
        y1 = pipe.forward(0, x)
        gemm()
        y2 = pipe.forward(1, y1)
        steps.append((ids, x, y1.clone(), y2.clone()))
        for i in range(2):
            rows, hit = pipe.stats(i)
            assert 0 <= hit <= rows and (cached or hit == 0), (s, i, rows, hit)
            served += hit
    torch.cuda.synchronize()
    assert (served > 0) == cached
    print(f"{len(steps)} steps issued without host synchronisation (cache {cached})", flush=True)

    for s, (ids, x, y1, y2) in enumerate(steps):
        dids = torch.from_numpy(ids).cuda()
        r1 = L[0]["plan"].forward(x, dids, L[0]["WK"], L[0]["WV"], L[0]["W_up"], L[0]["gamma"],
                                  L[0]["beta"], L[0]["W_mix"])
        r2 = L[1]["plan"].forward(y1, dids, L[1]["WK"], L[1]["WV"], L[1]["W_up"], L[1]["gamma"],
                                  L[1]["beta"], L[1]["W_mix"])
        assert torch.equal(y1, r1), f"step {s}: layer 1 differs from the resident forward"
        assert torch.equal(y2, r2), f"step {s}: layer 2 differs from the resident forward"
        if s in (0, 2, 4):
            n = len(ids)
            for case, xin, got, name in ((c1, x, y1, "layer 1"), (c2, y1, y2, "layer 2")):
                xin_bits = xin.view(torch.int16).cpu().numpy().view(np.uint16)
                ref = oracle_out(dataclasses.replace(case, ids=ids), x=xin_bits)
                err = rowwise_err(to_np(got), ref)
                print(f"step {s} ({n} tokens) {name} vs oracle: err {err:.2e}", flush=True)
                assert err <= case.tol
    pipe.close()
    for lay in L:
        lay["plan"].close()
