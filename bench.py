"""Benchmark of the L^3 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload paper_bf16] [--backward]

One step = one l3_forward over the whole batch (route, gather-attention, W_up,
W_mix) with every input already resident in HBM; the 256 MB MALL is flushed
before each timed step.  Prints one JSON line: tokens/s over K timed steps (HIP
events around each forward), the roofline of the dominant kernel (algorithmic
bytes or FLOPs per launch over its HIP-event duration, measured inside the
library on the launch stream), all stage rooflines, and the fp64 oracle timed
on a bounded token sample on the host cores.  `--backward` times l3_backward (the
training pass) the same way; `--workload decode_bf16` times decode steps with the
tables in pinned host memory.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TF = 2500.0  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TF = 157.3   # MI355X fp32 vector FMA
# the library's timed stages.  ln_stats_gemm: LayerNorm's row statistics, from the
# quadratic form o^T G o (a GEMM against G = W_c^T W_c and a finalize) above 512 tokens,
# from the W_up GEMM at or below; mix_prep: the weight-only factors F and G (above 512
# tokens) or the split-K W_up (at or below).
STAGES = ["route", "gather_mfma", "gather_light", "ln_stats_gemm", "mix_prep", "w_mix_gemm"]
# the source files a stage's kernels come from (a counter summary holds while they hash
# to the value recorded with it)
_HDRS = ("l3_internal.h", "cdna4.h")  # constants and helpers every kernel source includes
KERNEL_SOURCES = {"gather_attention": ("attn.hip",) + _HDRS, "gather_mfma": ("attn.hip",) + _HDRS,
                  "gather_light": ("attn.hip",) + _HDRS, "ln_stats_gemm": ("gemm.hip",) + _HDRS,
                  "mix_prep": ("gemm.hip", "gemm_skinny.hip", "backward.hip") + _HDRS,
                  "w_mix_gemm": ("gemm.hip",) + _HDRS, "route": ("route.hip",) + _HDRS}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; a decode workload's own step count)")
    # the first 20 or so forwards of a process run about 5 % slower than the rest (the
    # GPU settling after start-up), so the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="paper_bf16")
    ap.add_argument("--cache-rows", type=int, default=0,
                    help="decode: keep the rows of the most frequent IDs (up to this many rows) in a "
                         "device-resident cache")
    ap.add_argument("--layers", type=int, default=1, choices=(1, 2),
                    help="decode: also time a two-layer pipeline (both prefetches issued at step start)")
    ap.add_argument("--backward", action="store_true",
                    help="time l3_backward (the training pass) instead of the forward")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the oracle timing on the host")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-probe", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB (5 times) and exit: the "
                         "reference kernel that scales the HBM byte counters")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                           "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE of this "
                         "benchmark and of --copy-probe) into profiles/<stage>_<workload>_"
                         "counters.json, then exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size the copy probe ran with")
    ap.add_argument("--ingest-mfma", metavar="MFMA_CSV",
                    help="turn a rocprofv3 --pmc CSV of the MFMA counters into "
                         "profiles/<stage>_<workload>_mfma.json, then exit")
    args = ap.parse_args()
    args.steps_given = args.steps is not None
    if args.steps is None:
        args.steps = 50
    return args


def src_hash(names) -> str:
    """sha256 (first 16 hex digits) of the named sources' bytes, concatenated in order."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "static_token_routed_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(stage: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"{stage}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != src_hash(KERNEL_SOURCES[stage]):
        return None
    return d.get("hbm_bytes_per_launch")


def copy_probe(mib: int):
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[copy-probe] 5 copies of {mib} MiB done", file=sys.stderr, flush=True)


# kernel name prefix -> stage of one forward
STAGE_OF_KERNEL = [("k_attn_mfma", "gather_mfma"), ("k_attn_light", "gather_light"),
                   ("k_gemm_bf16<false, false, 3,", "ln_stats_gemm"),
                   ("k_gemm_bf16<true, false, 0,", "w_mix_gemm"),
                   ("k_transpose", "mix_prep"), ("k_center_rows", "mix_prep"), ("k_mix_fold", "mix_prep"),
                   ("k_gemm_bf16<false, false, 0,", "mix_prep"),  # [F ; G] (the only plain GEMM)
                   ("k_gemm_skinny", "mix_prep"), ("k_skinny_reduce", "mix_prep"),
                   ("k_sort", "route"), ("k_hist_scan", "route"), ("k_seg", "route"),
                   ("k_worklist", "route"), ("k_zero_i32", "route"), ("k_route_small", "route")]
COMPOSITE = {"gather_attention": ("gather_mfma", "gather_light")}


def read_counter_csv(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 CSV."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].replace("l3::(anonymous namespace)::", "").replace("l3::", "")
            name = name[5:] if name.startswith("void ") else name
            name = name.split("(")[0]
            per.setdefault(name, []).append(float(r["Counter_Value"]))
    return per


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8


def ingest_mfma(args):
    """MFMA utilisation of the two GEMM stages from one rocprofv3 --pmc run of
    SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: per
    dispatch, bf16 MFMA FLOP = MOPS x 512, busy fraction = busy cycles summed over the
    SIMDs / (GUI-active cycles per XCD x SIMDs), clock = GUI-active cycles per XCD /
    dispatch duration.  Means over the dispatches go to profiles/<stage>_<workload>_mfma.json."""
    import csv
    per = {}
    for r in csv.DictReader(open(args.ingest_mfma)):
        name = r["Kernel_Name"].replace("l3::(anonymous namespace)::", "").replace("l3::", "")
        name = (name[5:] if name.startswith("void ") else name).split("(")[0]
        key = (name, r["Dispatch_Id"])
        d = per.setdefault(key, {"dur_ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    stages = {}
    for (name, _), d in per.items():
        st = next((s_ for p_, s_ in STAGE_OF_KERNEL if name.startswith(p_)), None)
        if st not in ("ln_stats_gemm", "w_mix_gemm") or not all(c in d for c in MFMA_COUNTERS):
            continue
        gui = d["GRBM_GUI_ACTIVE"] / XCDS
        stages.setdefault(st, []).append({
            "flop": d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
            "busy": d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS),
            "clock_ghz": gui / d["dur_ns"], "dur_us": d["dur_ns"] / 1e3, "kernel": name})
    for st, rows in stages.items():
        out = {"stage": st, "workload": args.workload,
               "source_sha256_16": src_hash(KERNEL_SOURCES[st]), "kernel": rows[0]["kernel"],
               "dispatches": len(rows),
               "mfma_flop_per_launch": float(np.mean([r["flop"] for r in rows])),
               "mfma_busy_fraction": float(np.mean([r["busy"] for r in rows])),
               "clock_ghz": float(np.median([r["clock_ghz"] for r in rows])),
               "duration_us_mean": float(np.mean([r["dur_us"] for r in rows])),
               "commands": [" ".join(sys.argv)]}
        path = os.path.join(ROOT, "profiles", f"{st}_{args.workload}_mfma.json")
        json.dump(out, open(path, "w"), indent=1)
        print(f"{path}: busy {out['mfma_busy_fraction']:.3f}, {out['mfma_flop_per_launch'] / 1e9:.2f} "
              f"GFLOP, clock {out['clock_ghz']:.2f} GHz")


def mfma_from_profiles(stage: str, workload: str):
    """The counter-based MFMA figures of a GEMM stage, if taken on the current source."""
    p = os.path.join(ROOT, "profiles", f"{stage}_{workload}_mfma.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != src_hash(KERNEL_SOURCES[stage]):
        return None
    return {"busy_fraction": d["mfma_busy_fraction"], "flop_per_launch": d["mfma_flop_per_launch"],
            "clock_ghz": d["clock_ghz"],
            "source": f"profiles/{stage}_{workload}_mfma.json (rocprofv3 counters)"}


def ingest_counters(args):
    """HBM bytes per launch of each stage: mean per dispatch of FETCH_SIZE and
    WRITE_SIZE (KiB), each scaled by bytes / counter of the plain copy kernel."""
    fetch = read_counter_csv(args.ingest_counters[0], "FETCH_SIZE")
    write = read_counter_csv(args.ingest_counters[1], "WRITE_SIZE")
    cfetch = read_counter_csv(args.ingest_counters[2], "FETCH_SIZE")
    cwrite = read_counter_csv(args.ingest_counters[3], "WRITE_SIZE")
    copy_bytes = args.copy_mib << 20

    def copy_factor(per):
        k = max(per, key=lambda n: np.mean(per[n]))  # the copy kernel: largest reading
        return copy_bytes / (np.median(per[k]) * 1024.0), k

    ff, fk = copy_factor(cfetch)
    wf, wk = copy_factor(cwrite)
    stages = {}
    for name in fetch:
        st = next((s for p, s in STAGE_OF_KERNEL if name.startswith(p)), None)
        if st is None:
            continue
        d = stages.setdefault(st, {"kernels": {}, "fetch_kib": 0.0, "write_kib": 0.0})
        # per forward: dispatches of a kernel per forward = calls / forwards
        d["kernels"][name] = {"fetch_kib_per_dispatch": float(np.mean(fetch[name])),
                              "write_kib_per_dispatch": float(np.mean(write.get(name, [0.0]))),
                              "dispatches": len(fetch[name])}
    forwards = max(len(fetch[n]) for n in fetch if n.startswith("k_attn"))
    for st, d in stages.items():
        for name, kd in d["kernels"].items():
            per_fwd = kd["dispatches"] / forwards
            d["fetch_kib"] += kd["fetch_kib_per_dispatch"] * per_fwd
            d["write_kib"] += kd["write_kib_per_dispatch"] * per_fwd
    for comp, parts in COMPOSITE.items():
        d = stages.setdefault(comp, {"kernels": {}, "fetch_kib": 0.0, "write_kib": 0.0})
        for part in parts:
            if part in stages:
                d["kernels"].update(stages[part]["kernels"])
                d["fetch_kib"] += stages[part]["fetch_kib"]
                d["write_kib"] += stages[part]["write_kib"]
    for st, d in stages.items():
        out = {
            "stage": st, "workload": args.workload,
            "source_sha256_16": src_hash(KERNEL_SOURCES[st]),
            "fetch_kib_per_launch": d["fetch_kib"], "write_kib_per_launch": d["write_kib"],
            "copy_probe": {"bytes": copy_bytes, "fetch_kernel": fk, "write_kernel": wk,
                           "fetch_factor": ff, "write_factor": wf},
            "hbm_read_bytes_per_launch": d["fetch_kib"] * 1024.0 * ff,
            "hbm_write_bytes_per_launch": d["write_kib"] * 1024.0 * wf,
            "kernels": d["kernels"],
            "forwards_profiled": forwards,
            "commands": [" ".join(sys.argv)],
        }
        out["hbm_bytes_per_launch"] = out["hbm_read_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
        path = os.path.join(ROOT, "profiles", f"{st}_{args.workload}_counters.json")
        json.dump(out, open(path, "w"), indent=1)
        print(f"{path}: {out['hbm_bytes_per_launch'] / 1e9:.3f} GB per launch")


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args)
        return
    if args.ingest_mfma:
        ingest_mfma(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import synth
    import static_token_routed_amd as l3

    cfg = synth.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    if cfg.steps:
        decode_bench(args, cfg, torch, l3, synth)
        return
    if args.backward:
        backward_bench(args, cfg, torch, l3, synth)
        return
    t0 = time.time()
    off = synth.offsets(cfg)
    ids = synth.token_ids(cfg)
    x, WK, WV = synth.hidden(cfg), synth.table(cfg, "W_K"), synth.table(cfg, "W_V")
    Wup, Wmix = synth.dense(cfg, "W_up"), synth.dense(cfg, "W_mix")
    g, b = synth.ln_params(cfg)

    is32 = cfg.dtype == "f32"

    def dev(a):
        if is32:
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    dx, dWK, dWup, dWmix = dev(x), dev(WK), dev(Wup), dev(Wmix)
    # tied configuration: one device table serves as W_K and W_V
    dWV = dWK if cfg.tied else dev(WV)
    dids = torch.from_numpy(ids).cuda()
    dg, db = torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda()
    print(f"[bench] {cfg.name}: inputs generated and uploaded in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)

    plan = l3.L3Plan(off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, cfg.dtype, cfg.ln_eps)
    n = cfg.n
    out = torch.empty((n, cfg.d_out), dtype=torch.float32 if is32 else torch.bfloat16, device="cuda")
    ws = plan.workspace(n)

    def step():
        l3.l3_forward(plan.handle, dx, dids, n, dWK, dWV, dWup, dg, db, dWmix, out, ws, ws.numel())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert plan.status() == l3.L3_OK

    # Timed steps.  Before each forward the 256 MB MALL is flushed by a read-modify-
    # write of 512 MiB, so no step finds the previous step's rows (the Zipf head) in
    # it; each forward is timed by HIP events on its own stream, the flush is not.
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in ev:
        flush_buf.add_(1)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    fwd_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    elapsed = sum(fwd_ms) * 1e-3
    print(f"[bench] {args.steps} flushed steps: {elapsed * 1e3:.3f} ms of forward time "
          f"({wall:.4f}s wall with the flushes)", file=sys.stderr, flush=True)

    # steady state without the flushes (context: the MALL then holds the hottest rows)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    warm = (time.perf_counter() - t0) / args.steps

    # per-kernel times: the same number of flushed steps again, with the library's HIP
    # events around each kernel stage on the launch stream
    l3.l3_profile_enable(True)
    for _ in range(args.steps):
        flush_buf.add_(1)
        step()
    stage_ms, launches = l3.l3_profile_read(len(STAGES))
    del flush_buf
    l3.l3_profile_enable(False)

    # algorithmic work per launch: distinct K/V rows (split by the library's work-list
    # rule between the two gather-attention kernels) and dense FLOPs
    u, cnt = np.unique(ids, return_counts=True)
    d = off[u + 1] - off[u]
    min_tok, min_rows = l3.l3_worklist_rule(plan.handle)
    heavy = (cnt >= min_tok) | (d >= min_rows)
    # a tied configuration's row serves both roles: its algorithmic bytes are one row
    row_b = (cfg.d_in + (0 if cfg.tied else cfg.d_emb)) * (4 if is32 else 2)
    R = int(d.sum())
    kv = {"gather_attention": R * row_b, "gather_mfma": int(d[heavy].sum()) * row_b,
          "gather_light": int(d[~heavy].sum()) * row_b}
    # batches of more than 512 tokens run W_mix factored through W_up: one GEMM over
    # [o | x] (K = d_emb + d_in) against [F | W2], F = W1 diag(gamma) W_c, and
    # LayerNorm's variance from o^T G o (GEMM o G, N = K = d_emb), F and G formed per
    # call in the preparation stage; smaller batches run W_up and W_mix over [LN(h) | x]
    factored = n > 512 and not is32
    up_flops = 2.0 * n * cfg.d_emb * (cfg.d_emb if factored else cfg.d_up)
    mix_k = (cfg.d_emb + cfg.d_in) if factored else (cfg.d_up + cfg.d_in)
    mix_flops = 2.0 * n * cfg.d_out * mix_k
    avg = {s_: stage_ms[i] / max(1, launches[i]) for i, s_ in enumerate(STAGES)}
    avg["gather_attention"] = avg["gather_mfma"] + avg["gather_light"]
    kernels = {}
    for k_ in ("gather_attention", "gather_mfma", "gather_light"):
        rows = kv[k_] // row_b
        kernels[k_] = {"bound": "hbm", "achieved": kv[k_] / (avg[k_] * 1e-3) / 1e9 if avg[k_] else 0.0,
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "work_per_launch": f"{kv[k_]} B of distinct K/V rows ({rows} rows x {row_b} B)"}
    kernels["gather_attention"]["kernels"] = "gather_mfma + gather_light"
    # fp32 plans run their GEMMs on the vector ALUs (fp32 FMA peak 157.3 TFLOP/s)
    gemm_bound, gemm_peak = ("alu", FP32_VALU_PEAK_TF) if is32 else ("mfma", MFMA_BF16_PEAK_TF)
    kernels["ln_stats_gemm"] = {"bound": gemm_bound,
                                "achieved": up_flops / (avg["ln_stats_gemm"] * 1e-3) / 1e12,
                                "peak": gemm_peak, "unit": "TFLOP/s",
                                "work_per_launch": f"{up_flops:.4g} FLOP ("
                                + ("o G, K = N = d_emb" if factored else "W_up, K = d_emb") + ")"}
    kernels["w_mix_gemm"] = {"bound": gemm_bound, "achieved": mix_flops / (avg["w_mix_gemm"] * 1e-3) / 1e12,
                             "peak": gemm_peak, "unit": "TFLOP/s",
                             "work_per_launch": f"{mix_flops:.4g} FLOP (K = {mix_k})"}
    for k_, v_ in kernels.items():
        v_["frac"] = v_["achieved"] / v_["peak"]
        v_["ms"] = avg[k_]
        v_["traffic"] = traffic_from_profiles(k_, cfg.name)
    for k_ in ("ln_stats_gemm", "w_mix_gemm"):
        kernels[k_]["mfma_counters"] = mfma_from_profiles(k_, cfg.name)
    # the dominant single kernel (longest average launch)
    dominant = max(("gather_mfma", "gather_light", "ln_stats_gemm", "w_mix_gemm"), key=lambda s_: avg[s_])
    roof = {k_: kernels[dominant][k_] for k_ in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dominant

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, off, ids, x, WK, WV, Wup, Wmix, g, b, args.cpu_seconds)

    ms_per_step = elapsed / args.steps * 1e3
    line = {
        "metric": "L3 fwd tokens/s; K/V gather GB/s vs HBM peak; MFMA util (v=710K, d_in=2048)",
        "value": n * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Zipf token IDs, Zipf-shaped allocation, N(0, 1/sqrt(fan_in)) weights)",
        "config": {"workload": f"{cfg.name}: vocab {cfg.vocab}, v {cfg.v}, k {cfg.k}, d_in {cfg.d_in}, "
                               f"d_emb {cfg.d_emb}, d_up {cfg.d_up}, d_out {cfg.d_out}, "
                               f"{n} tokens, token IDs Zipf({cfg.ids_s})",
                   "global_batch": n, "distinct_ids": int(len(u)), "distinct_rows": R},
        "roofline": roof,
        "kernels": kernels,
        "stage_ms": {s_: avg[s_] for s_ in STAGES},
        "timing": {"method": "HIP events around each forward, MALL flushed (512 MiB read-modify-write) "
                             "before each; value and ms_per_step are their mean",
                   "ms_median": float(np.median(fwd_ms)), "ms_min": float(min(fwd_ms)),
                   "ms_max": float(max(fwd_ms)),
                   "unflushed_ms_per_step": warm * 1e3, "unflushed_tokens_per_s": n / warm},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    plan.close()


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def decode_bench(args, cfg, torch, l3, synth):
    """Decode steps with the tables in pinned host memory.

    A step starts when its token IDs are known: l3_prefetch copies the distinct
    rows of the step's IDs to the device on a side stream while a synthetic pre-layer
    GEMM (pre_m x pre_k x pre_n) runs on the main stream; the main stream then waits
    for the copies and runs l3_forward_staged; the step ends when its output is ready
    (host synchronisation, as sampling the next token needs it).  The same steps are
    also timed with the copy alone, the GEMM alone and copy + GEMM together, which
    gives the overlap ov = t_copy + t_gemm - t_concurrent.
    """
    n = cfg.n
    S = args.steps if args.steps_given else cfg.steps
    off = synth.offsets(cfg)
    ids = [synth.token_ids(cfg, step=s_) for s_ in range(S)]
    WK, WV = synth.table(cfg, "W_K"), synth.table(cfg, "W_V")

    def pinned(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).pin_memory()

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    WKh, WVh = pinned(WK), pinned(WV)
    del WK, WV
    x = dev(synth.hidden(cfg))
    Wup, Wmix = dev(synth.dense(cfg, "W_up")), dev(synth.dense(cfg, "W_mix"))
    g, b = (torch.from_numpy(a).cuda() for a in synth.ln_params(cfg))
    pa, pb = (dev(a) for a in synth.pre_gemm_operands(cfg))
    pc = torch.empty((cfg.pre_m, cfg.pre_n), dtype=torch.bfloat16, device="cuda")
    pws = torch.empty(max(16, l3.l3_gemm_workspace_size(cfg.pre_m, cfg.pre_n, cfg.pre_k)),
                      dtype=torch.uint8, device="cuda")
    plan = l3.L3Plan(off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, "bf16", cfg.ln_eps)
    out = torch.empty((n, cfg.d_out), dtype=torch.bfloat16, device="cuda")
    ws = plan.workspace(n)
    st = l3.l3_staging_create(plan.handle, n * cfg.k, n)
    # hot-row cache: the token stream is Zipf over the IDs in rank order, so the most
    # frequent IDs are 0, 1, 2, ...; keep whole IDs until the row budget is used
    dts = np.diff(off)
    hot = np.arange(int(np.searchsorted(np.cumsum(dts), args.cache_rows, side="right")), dtype=np.int32)
    if len(hot):
        l3.l3_staging_set_cache(st, hot, WKh, WVh)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()

    def prefetch(s_):
        l3.l3_prefetch(plan.handle, ids[s_], n, WKh, WVh, st, side, ready)

    def gemm():
        l3.l3_gemm_bf16(pa, pb, pc, cfg.pre_m, cfg.pre_n, cfg.pre_k, pws, pws.numel())

    def forward():
        l3.l3_forward_staged(st, x, n, Wup, g, b, Wmix, out, ws, ws.numel())

    def full(s_):
        prefetch(s_)
        gemm()
        main.wait_stream(side)
        forward()
        main.synchronize()

    staged = {}

    def copy_only(s_):
        prefetch(s_)
        ready.synchronize()
        staged[s_] = l3.l3_staging_stats(st)

    def gemm_only(s_):
        gemm()
        main.synchronize()

    def concurrent(s_):
        prefetch(s_)
        gemm()
        ready.synchronize()
        main.synchronize()

    def timed(fn):
        t = np.empty(S)
        for s_ in range(S):
            t0 = time.perf_counter()
            fn(s_)
            t[s_] = time.perf_counter() - t0
        return t * 1e6

    for _ in range(max(1, args.warmup)):
        for fn in (full, copy_only, gemm_only, concurrent):
            fn(0)
    torch.cuda.synchronize()
    t_step = timed(full)
    t_copy = timed(copy_only)
    t_gemm = timed(gemm_only)
    t_conc = timed(concurrent)
    prefetch(S - 1)
    ready.synchronize()
    t_fwd = timed(lambda s_: (forward(), main.synchronize()))
    assert plan.status() == l3.L3_OK

    rows = np.array([int(dts[np.unique(i)].sum()) for i in ids])
    cached = np.array([int(dts[np.intersect1d(np.unique(i), hot)].sum()) for i in ids])
    # the library's own count of staged and cache-served rows must agree
    assert all(staged[s_] == (rows[s_], cached[s_]) for s_ in range(S)), "staging stats disagree"
    row_b = (cfg.d_in + cfg.d_emb) * 2
    cfrac = float(cached.sum() / rows.sum())
    h2d = (rows - cached) * row_b
    pipe = decode_pipeline2(args, cfg, torch, l3, synth, ids, hot, WKh, WVh, x, Wup, g, b, Wmix, gemm,
                            timed) if args.layers == 2 else None
    med = lambda a: float(np.median(a))
    ov = med(t_copy) + med(t_gemm) - med(t_conc)
    pcie = float(h2d.mean()) / (med(t_copy) * 1e-6) / 1e9
    l3.l3_staging_destroy(st)
    plan.close()
    line = {
        "metric": "L3 decode step latency (pinned-host tables, prefetch overlapped with a pre-layer GEMM)",
        "value": n / (t_step.mean() * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": S, "warmup": args.warmup,
        "ms_per_step": float(t_step.mean()) * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf token IDs per step, Zipf-shaped allocation, N(0, 1/sqrt(fan_in)) weights)",
        "config": {"workload": f"{cfg.name}: vocab {cfg.vocab}, v {cfg.v}, k {cfg.k}, d_in {cfg.d_in}, "
                               f"d_emb {cfg.d_emb}, d_up {cfg.d_up}, d_out {cfg.d_out}, {n} tokens per "
                               f"step, tables in pinned host memory, pre-layer GEMM {cfg.pre_m}x"
                               f"{cfg.pre_k}x{cfg.pre_n}",
                   "global_batch": n},
        "roofline": {"bound": "pcie", "achieved": pcie, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": pcie / PCIE_PEAK_GBS, "traffic": None, "kernel": "l3_prefetch copies",
                     "work_per_launch": f"{h2d.mean():.4g} B of distinct K/V rows per step (mean)"},
        "decode": {
            "t_step_us": {"median": med(t_step), "p99": float(np.percentile(t_step, 99)),
                          "mean": float(t_step.mean())},
            "t_copy_us": med(t_copy), "t_gemm_us": med(t_gemm), "t_concurrent_us": med(t_conc),
            "t_forward_staged_us": med(t_fwd),
            "overlap_us": ov, "f_copy_hidden": ov / med(t_copy), "f_gemm_covered": ov / med(t_gemm),
            "rows_per_step": {"mean": float(rows.mean()), "max": int(rows.max())},
            "h2d_bytes_per_step": float(h2d.mean()),
            "cache": {"rows": int(dts[hot].sum()) if len(hot) else 0, "ids": int(len(hot)),
                      "fraction_of_step_rows_served": cfrac},
            "pipeline_2layer": pipe,
            "timing": "host clock from issuing the step's work to its synchronisation; medians "
                      "over the steps unless named",
        },
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_bench(args, cfg, torch, l3, synth):
    """Backward (training) pass: gradients of sum(dout * L3(x, ids)) for one batch, fp32
    gradients; dW_K / dW_V accumulate into full-size fp32 tables.  Timed like the
    forward (HIP events, last-level cache flushed before each step)."""
    t0 = time.time()
    off, ids = synth.offsets(cfg), synth.token_ids(cfg)
    x, WK, WV = synth.hidden(cfg), synth.table(cfg, "W_K"), synth.table(cfg, "W_V")
    Wup, Wmix = synth.dense(cfg, "W_up"), synth.dense(cfg, "W_mix")
    g, b = synth.ln_params(cfg)
    n, v = cfg.n, int(off[-1])

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    dout = torch.from_numpy(synth.f32_to_bf16_bits(
        np.random.default_rng(cfg.seed + 7).standard_normal((n, cfg.d_out), dtype=np.float32))
        .view(np.int16)).view(torch.bfloat16).cuda()
    args_in = [dev(x), torch.from_numpy(ids).cuda(), n, dev(WK), dev(WV), dev(Wup),
               torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(), dev(Wmix), dout]
    z = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device="cuda")
    grads = [z(n, cfg.d_in), z(v, cfg.d_in), z(v, cfg.d_emb), z(cfg.d_up, cfg.d_emb), z(cfg.d_up),
             z(cfg.d_up), z(cfg.d_out, cfg.d_up + cfg.d_in)]
    plan = l3.L3Plan(off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, "bf16", cfg.ln_eps)
    ws = torch.empty(l3.l3_backward_workspace_size(plan.handle, n), dtype=torch.uint8, device="cuda")
    print(f"[bench] {cfg.name} backward: inputs ready in {time.time() - t0:.1f}s, workspace "
          f"{ws.numel() / 1e9:.2f} GB", file=sys.stderr, flush=True)

    def step():
        l3.l3_backward(plan.handle, *args_in, *grads, ws, ws.numel())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        flush_buf.add_(1)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    l3.l3_profile_enable(True)
    for _ in range(args.steps):
        flush_buf.add_(1)
        step()
    st_ms, launches = l3.l3_profile_read(10)
    l3.l3_profile_enable(False)
    del flush_buf
    assert l3.l3_status(ws) == l3.L3_OK  # the route's flag, in the backward workspace
    names = {0: "route", 1: "gather_mfma", 2: "gather_light", 6: "recompute_h", 7: "dense_bwd",
             8: "attn_bwd", 9: "kv_grad"}
    avg = {nm: st_ms[i] / max(1, launches[i]) for i, nm in names.items()}
    # algorithmic bytes (both kernels are bound by memory traffic, not arithmetic):
    # the attention backward reads each distinct K / V row once, each token's x row,
    # dO (fp32) and o (bf16), and adds its term to dx (fp32, read + write); the key /
    # value gradients add into the fp32 gradient rows of the batch's distinct rows
    # (read + write) from each token's x row and dO row.
    tok_rows = float((off[ids + 1] - off[ids]).sum())
    uids = np.unique(ids)
    rows = float((off[uids + 1] - off[uids]).sum())
    attn_b = rows * (cfg.d_in + cfg.d_emb) * 2 + n * (cfg.d_in * 2 + cfg.d_emb * 6 + cfg.d_in * 8)
    kv_b = rows * (cfg.d_in + cfg.d_emb) * 8 + n * (cfg.d_in * 2 + cfg.d_emb * 4)
    Z = cfg.d_up + cfg.d_in
    dense_fl = 2.0 * n * (2 * cfg.d_out * Z + 2 * cfg.d_up * cfg.d_emb)
    kernels = {
        "attn_bwd": {"bound": "hbm", "achieved": attn_b / (avg["attn_bwd"] * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "work_per_launch": f"{attn_b:.4g} B ({rows:.0f} distinct K/V rows once, x, dO, o, "
                                        f"dx read + write; {tok_rows:.4g} token-rows)"},
        "kv_grad": {"bound": "hbm", "achieved": kv_b / (avg["kv_grad"] * 1e-3) / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "work_per_launch": f"{kv_b:.4g} B (fp32 gradient rows of {rows:.0f} distinct rows "
                                       f"read + written, x and dO once)"},
        "dense_bwd": {"bound": "mfma", "achieved": dense_fl / (avg["dense_bwd"] * 1e-3) / 1e12,
                      "peak": MFMA_BF16_PEAK_TF, "unit": "TFLOP/s",
                      "work_per_launch": f"{dense_fl:.4g} FLOP (dz, dW_mix, dW_up, do GEMMs; "
                                         f"transposes and LayerNorm backward in the same stage)"},
    }
    for k_, v_ in kernels.items():
        v_["frac"] = v_["achieved"] / v_["peak"]
        v_["ms"] = avg[k_]
        v_["traffic"] = None
    dominant = max(kernels, key=lambda k_: kernels[k_]["ms"])
    roof = {k_: kernels[dominant][k_] for k_ in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dominant
    mean = float(np.mean(ms))
    line = {
        "metric": "L3 backward tokens/s (fp32 gradients of x, W_K, W_V, W_up, LayerNorm, W_mix)",
        "value": n / (mean * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": mean, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf token IDs, Zipf-shaped allocation, N(0, 1/sqrt(fan_in)) "
                "weights, N(0, 1) upstream gradient)",
        "config": {"workload": f"{cfg.name}: vocab {cfg.vocab}, v {cfg.v}, k {cfg.k}, d_in {cfg.d_in}, "
                               f"d_emb {cfg.d_emb}, d_up {cfg.d_up}, d_out {cfg.d_out}, {n} tokens",
                   "global_batch": n},
        "roofline": roof, "kernels": kernels, "stage_ms": avg,
        "timing": {"method": "HIP events around each backward, MALL flushed before each",
                   "ms_median": float(np.median(ms)), "ms_min": float(min(ms)), "ms_max": float(max(ms))},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    plan.close()


def decode_pipeline2(args, cfg, torch, l3, synth, ids, hot, WKh1, WVh1, x, Wup1, g1, b1, Wmix1,
                     gemm, timed):
    """Two lookup layers per decode step, as the pages place L^3 after several decoder
    layers, through l3.DecodeLayers (the path tests/test_gpu_decode_pipeline.py checks
    bit for bit): both layers' prefetches are issued when the step starts, each on its
    own side stream and staging (layer 2 with its own tables), then the main stream
    runs the pre-layer GEMM, layer 1, the same GEMM again for the layers in between,
    and layer 2 (whose input is layer 1's output).  t_copies: both prefetches alone;
    t_compute: the same step with its rows already staged; ov = t_copies + t_compute -
    t_step."""
    n = cfg.n
    assert cfg.d_out == cfg.d_in, "layer 2 reads layer 1's output"
    c2 = dataclasses.replace(cfg, seed=cfg.seed + 1)

    def pinned(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).pin_memory()

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    off = synth.offsets(cfg)
    mk = lambda: l3.L3Plan(off, cfg.k, cfg.d_in, cfg.d_emb, cfg.d_up, cfg.d_out, "bf16", cfg.ln_eps)
    layers = [
        {"plan": mk(), "W_K_host": WKh1, "W_V_host": WVh1, "W_up": Wup1, "gamma": g1, "beta": b1,
         "W_mix": Wmix1},
        {"plan": mk(), "W_K_host": pinned(synth.table(c2, "W_K")),
         "W_V_host": pinned(synth.table(c2, "W_V")), "W_up": dev(synth.dense(c2, "W_up")),
         "gamma": g1, "beta": b1, "W_mix": dev(synth.dense(c2, "W_mix"))},
    ]
    pipe = l3.DecodeLayers(layers, max_tokens=n)
    if len(hot):
        pipe.set_cache(0, hot)
        pipe.set_cache(1, hot)
    main = torch.cuda.current_stream()

    def compute():
        gemm()
        y1 = pipe.forward(0, x)
        gemm()
        pipe.forward(1, y1)

    def step(s_):
        pipe.prefetch(ids[s_])
        compute()
        main.synchronize()

    def copies(s_):
        pipe.prefetch(ids[s_])
        for lay in pipe.layers:
            lay["ready"].synchronize()

    def compute_only(s_):
        compute()
        main.synchronize()

    for _ in range(max(1, args.warmup)):
        step(0)
    t_step, t_cp = timed(step), timed(copies)
    t_cmp = timed(compute_only)
    pipe.close()
    for lay in layers:
        lay["plan"].close()
    med = lambda a: float(np.median(a))
    ov = med(t_cp) + med(t_cmp) - med(t_step)
    return {"t_step_us": {"median": med(t_step), "p99": float(np.percentile(t_step, 99)),
                          "mean": float(t_step.mean())},
            "t_copies_us": med(t_cp), "t_compute_us": med(t_cmp), "overlap_us": ov,
            "f_copy_hidden": ov / med(t_cp),
            "tokens_per_s": n / (float(t_step.mean()) * 1e-6)}


def cpu_baseline(cfg, off, ids, x, WK, WV, Wup, Wmix, g, b, seconds):
    """The fp64 oracle as it stands, on a seeded sample of the batch's tokens,
    grown until about `seconds` of wall time; tokens/s over the timed chunks."""
    import oracle

    f32 = lambda a: synth_f32(a, cfg.dtype)
    nt = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(123)
    order = rng.permutation(len(ids))
    Wup64, Wmix64 = f32(Wup).astype(np.float64), f32(Wmix).astype(np.float64)
    done, spent, chunk = 0, 0.0, 64
    while spent < seconds and done < len(ids):
        rows = order[done:done + chunk]
        u, inv = np.unique(ids[rows], return_inverse=True)
        dd = off[u + 1] - off[u]
        coff = np.concatenate([[0], np.cumsum(dd)]).astype(np.int64)
        sel = np.concatenate([np.arange(off[t], off[t + 1]) for t in u])
        xs, wk, wv = f32(x[rows]), f32(WK[sel]), f32(WV[sel])
        t = time.perf_counter()
        oracle.forward(coff, cfg.k, xs, inv.astype(np.int32), wk, wv, Wup64, g, b, Wmix64,
                       eps=cfg.ln_eps, nthreads=nt)
        spent += time.perf_counter() - t
        done += len(rows)
        chunk = min(chunk * 2, 1024)
    # one thread, a seeded 512-token sample (the first tokens of the same permutation)
    rows = order[:512]
    u, inv = np.unique(ids[rows], return_inverse=True)
    dd = off[u + 1] - off[u]
    coff = np.concatenate([[0], np.cumsum(dd)]).astype(np.int64)
    sel = np.concatenate([np.arange(off[t], off[t + 1]) for t in u])
    xs, wk, wv = f32(x[rows]), f32(WK[sel]), f32(WV[sel])
    t = time.perf_counter()
    oracle.forward(coff, cfg.k, xs, inv.astype(np.int32), wk, wv, Wup64, g, b, Wmix64,
                   eps=cfg.ln_eps, nthreads=1)
    one = len(rows) / (time.perf_counter() - t)
    return {"value": done / spent, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"{done} tokens drawn (seeded) from the {cfg.name} batch, tables cut to "
                      f"their rows; {spent:.1f}s of oracle time on {nt} threads",
            "single_thread": {"value": one, "unit": "tokens/s",
                              "sample": "512 tokens of the same seeded draw, 1 thread"},
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def synth_f32(a, dtype):
    import synth
    return synth.as_f32(a, dtype)


if __name__ == "__main__":
    main()
