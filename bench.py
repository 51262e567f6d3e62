"""Benchmark: SLA forward + backward at L = 16K on one MI355X.

One step is the whole hot path over one batch: the on-device tile schedule,
the forward, and the backward (gradient scale + schedule, dK/dV, dQ) of HSTU
SiLU attention under the semi-local mask, on the long_16k workload (B = 8,
lengths 16384 x 4 + U[4096, 16384] x 4, H = 4, d = 128, K1 = 1024, K2 = 128,
contextual 16, bf16, seed 0), inputs resident in HBM before timing starts.

Prints one JSON line: useful TFLOP/s (visible pairs only, 1792 flop per pair
per head), plus tokens/s, the roofline of the dominant kernel (per-kernel time
from HIP events recorded on the library's stream) and the fp64 CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0
WORKLOAD = "long_16k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=(WORKLOAD, "stu_layer", "stu_stack", "mfalcon",
                                           "targets_16k", "jagged_2k"),
                    default=WORKLOAD,
                    help="long_16k: the SLA forward + backward (default); stu_layer: one full "
                         "STU layer forward + backward at the 18-layer stack's shape; "
                         "stu_stack: the 18-layer STU stack forward; mfalcon: candidate "
                         "scoring against cached history keys/values; jagged_2k: the SLA "
                         "forward + backward at B=32, L U[512,2048], eager and as one HIP "
                         "graph replay")
    ap.add_argument("--fp8", action="store_true",
                    help="stu_stack: both projections of every layer in FP8")
    ap.add_argument("--candidates", type=int, default=4096,
                    help="mfalcon: candidates per sequence")
    ap.add_argument("--microbatch", type=int, default=1024,
                    help="mfalcon: candidates per sequence and call")
    ap.add_argument("--outputs", choices=("f32", "bf16"), default="f32",
                    help="long_16k: dtype of O, dQ, dK, dV (inputs are bf16 either way); f32 is "
                         "the configuration the parity tests hold to the stated bar")
    ap.add_argument("--dq", choices=("stored", "recompute"), default="stored",
                    help="long_16k: dQ from the dS the dK/dV kernel stores (default workspace), "
                         "or recomputed with the smallest workspace")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the MFMA-only probe (run after the timed steps) that reports the "
                         "bf16 MFMA rate and shader clock measured on this GPU")
    ap.add_argument("--issue-probe", action="store_true",
                    help="long_16k: after the timed steps, run the issue-rate probe (MFMA and "
                         "VALU overlap on one SIMD, transcendental cost) and add its durations")
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536,
                    help="cpu_baseline: whole sequences from the start of the workload up to "
                         "about this many tokens (long_16k: its four 16384-token sequences)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_long_16k.json"),
                    help="per-kernel HBM bytes measured with rocprofv3 --pmc (optional)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed steps, run a plain fp32 negation of 256 MiB (read and "
                         "written once) whose FETCH_SIZE / WRITE_SIZE calibrate the counters")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: read the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE csv "
                         "output of a --calibration-copy run and write --traffic")
    return ap.parse_args()


# kernels whose HBM traffic the bench line reports, by the name rocprofv3 gives them
PMC_KERNELS = {"fwd": "sla_fwd_bf16_kernel<128, 128, false",
               "bwd_dkdv": "sla_bwd_dkdv_bf16_kernel<128, 128",
               "bwd_dq": "sla_bwd_dq_stored_kernel<128"}
CALIB_BYTES = 256 * 1024 * 1024
CALIB_NAME = "neg_kernel_cuda"


def summarize_pmc(fetch_dir, write_dir, out):
    """Per-dispatch HBM bytes of the SLA kernels from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled so that the calibration negation of
    256 MiB reads and writes exactly 256 MiB."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024)
        return vals

    res = {"calibration": {"kernel": "torch.neg of 256 MiB fp32", "bytes": CALIB_BYTES}}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        vals = per_kernel(d, counter)
        cal = [v for k, vs in vals.items() if CALIB_NAME in k for v in vs]
        if not cal:
            raise SystemExit(f"no calibration dispatch in {d}")
        factor = CALIB_BYTES / (sum(cal) / len(cal))
        res["calibration"][f"{key}_scale"] = round(factor, 4)
        for short, name in PMC_KERNELS.items():
            vs = [v for k, vl in vals.items() if name in k for v in vl]
            if vs:
                res.setdefault(short, {})[f"{key}_bytes"] = int(factor * sum(vs) / len(vs))
    for short in PMC_KERNELS:
        if short in res and "fetch_bytes" in res[short] and "write_bytes" in res[short]:
            res[short]["hbm_bytes"] = res[short]["fetch_bytes"] + res[short]["write_bytes"]
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): there is no "
              "multi-GPU path to time; the attention would shard by sequence with no "
              "exchange, which nothing here runs or measures", file=sys.stderr)
        sys.exit(2)

    if args.workload == "stu_layer":
        bench_stu_layer(args)
        return
    if args.workload == "mfalcon":
        bench_mfalcon(args)
        return
    if args.workload == "stu_stack":
        bench_stu_stack(args)
        return
    if args.workload == "targets_16k":
        bench_targets_fwd(args)
        return
    if args.workload == "jagged_2k":
        bench_jagged_graph(args)
        return
    import torch
    import sparse_sequence_attention_amd as sla
    from synthetic import make_sla_workload, CONFIGS

    cfg = CONFIGS[WORKLOAD]
    w = make_sla_workload(cfg, seed=args.seed, with_dout=True)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = torch.bfloat16
    q, k, v, do = (torch.from_numpy(a).to(dev).to(dt) for a in (w.q, w.k, w.v, w.dout))
    offs = torch.from_numpy(w.offsets).to(dev)
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len)
    H, d = cfg.heads, cfg.d
    odt = torch.float32 if args.outputs == "f32" else dt
    o, dq, dk, dv = (torch.empty(q.shape, dtype=odt, device=dev) for _ in range(4))
    p = sla.make_problem(dt, offs, None, w.total_tokens, H, d, d, **kw)
    ws = torch.empty(max(sla.workspace_size(p, sla.SLA_OP_BWD),
                         sla.workspace_size(p, sla.SLA_OP_FWD)), dtype=torch.uint8, device=dev)

    recompute = args.dq == "recompute"

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sla.sla_fwd(q, k, v, offs, None, out=o, workspace=ws, **kw)
        if ev is not None:
            ev[1].record()
        sla.sla_bwd(q, k, v, do, offs, None, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stage=sla.SLA_BWD_PREPARE, recompute_dq=recompute, **kw)
        if ev is not None:
            ev[2].record()
        sla.sla_bwd(q, k, v, do, offs, None, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stage=sla.SLA_BWD_DKDV, recompute_dq=recompute, **kw)
        if ev is not None:
            ev[3].record()
        sla.sla_bwd(q, k, v, do, offs, None, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stage=sla.SLA_BWD_DQ, recompute_dq=recompute, **kw)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.calibration_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # medians over the timed steps
    ms_step = float(np.median([events[i][0].elapsed_time(events[i][4])
                               for i in range(args.steps)]))
    phase = {name: float(np.median([events[i][a].elapsed_time(events[i][b])
                                    for i in range(args.steps)]))
             for name, a, b in (("fwd", 0, 1), ("bwd_prepare", 1, 2), ("bwd_dkdv", 2, 3),
                                ("bwd_dq", 3, 4))}

    pairs = sla.count_pairs_host(w.offsets, None, w.k1, w.k2, w.contextual_len) * H
    useful = pairs * (2 * (d + d) + 2 * (3 * d + 2 * d))
    value = useful / (ms_step * 1e-3) / 1e12
    tokens_s = w.total_tokens / (ms_step * 1e-3)
    # algorithmic MFMA work of each kernel (per launch): forward S and P.V; dK/dV
    # kernel S, dP, dV, dK; dQ kernel dQ = dS K (from the stored dS by default;
    # with --dq recompute its recomputed S and dP are not counted)
    kernel_flops = {"fwd": pairs * 4 * d, "bwd_dkdv": pairs * 8 * d, "bwd_dq": pairs * 2 * d}
    dom = max(kernel_flops, key=lambda n: phase[n])
    achieved = kernel_flops[dom] / (phase[dom] * 1e-3) / 1e12
    traffic = None
    # the committed counters were taken on the default (stored-dS) backward
    if os.path.exists(args.traffic) and not (recompute and dom.startswith("bwd")):
        with open(args.traffic) as f:
            traffic = json.load(f).get(dom, {}).get("hbm_bytes")

    line = {
        "metric": "SLA fwd+bwd useful TFLOP/s & tokens/s at L=16K; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{WORKLOAD}: {cfg.description}, N={cfg.max_seq_len}, seed {args.seed}",
            "outputs": args.outputs, "dq": args.dq,
            "total_tokens": w.total_tokens,
            "visible_pairs_all_heads": pairs,
            "useful_flop_per_step": useful,
        },
        "tokens_per_s": round(tokens_s, 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "phase_ms": {kk: round(vv, 4) for kk, vv in phase.items()},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_peak_probe:
        # after the timed region: the MFMA-only rate and the shader clock on this GPU
        pm = sla.probe_mfma_peak()
        line["peak_measured"] = {
            "kernel": "MFMA-only: bf16 32x32x16, four independent chains per wave, 16 waves per CU",
            "tflops": round(pm["tflops"], 1),
            "sclk_ghz": round(pm["sclk_ghz"], 3),
            "pct_of_measured_peak": round(100.0 * value / pm["tflops"], 2),
            "roofline_frac_of_measured_peak": round(achieved / pm["tflops"], 4),
        }
    if args.issue_probe:
        ip = sla.probe_issue_rates()
        line["issue_probe"] = {k: round(v, 4) for k, v in ip.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    print(json.dumps(line), flush=True)


def bench_jagged_graph(args):
    """SLA forward + backward on the jagged_2k workload (B = 32, lengths
    U[512, 2048], H = 4, d = 128, K1 = 256, K2 = 64, ctx 8, fp32 outputs),
    whose steps are short enough for launch gaps to show: K steps issued
    eagerly, then the same step recorded once as a HIP graph (torch's
    CUDAGraph over the library's calls, outputs and workspace owned by the
    caller) and K replays.  Each run is bracketed by synchronisations and
    timed with events on the stream; value is the replayed rate."""
    import torch
    import sparse_sequence_attention_amd as sla
    from synthetic import make_sla_workload, CONFIGS

    cfg = CONFIGS["jagged_2k"]
    w = make_sla_workload(cfg, seed=args.seed, with_dout=True)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = torch.bfloat16
    q, k, v, do = (torch.from_numpy(a).to(dev).to(dt) for a in (w.q, w.k, w.v, w.dout))
    offs = torch.from_numpy(w.offsets).to(dev)
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len)
    H, d = cfg.heads, cfg.d
    o, dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(4))
    p = sla.make_problem(dt, offs, None, w.total_tokens, H, d, d, **kw, out_f32=True)
    ws = torch.empty(max(sla.workspace_size(p, sla.SLA_OP_BWD),
                         sla.workspace_size(p, sla.SLA_OP_FWD)), dtype=torch.uint8, device=dev)

    def step():
        sla.sla_fwd(q, k, v, offs, None, out=o, workspace=ws, **kw)
        sla.sla_bwd(q, k, v, do, offs, None, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    for _ in range(args.warmup):
        step()
    eager_ms = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    graph_ms = timed(g.replay)

    pairs = sla.count_pairs_host(w.offsets, None, w.k1, w.k2, w.contextual_len) * H
    useful = pairs * (2 * (d + d) + 2 * (3 * d + 2 * d))
    # compulsory HBM bytes of the step per token and head: the forward reads
    # q, k, v (bf16) and writes O (fp32); the backward reads q, k, v, dO and
    # writes dQ, dK, dV (fp32).  At K1 = 256 the arithmetic intensity is below
    # the ridge, so the step is rated against HBM bandwidth too.
    compulsory = w.total_tokens * H * ((3 * 2 * d + 4 * d) + (4 * 2 * d + 3 * 4 * d))
    hbm_gbs = compulsory / (graph_ms * 1e-3) / 1e9
    line = {
        "metric": "SLA fwd+bwd useful TFLOP/s (jagged_2k, eager and HIP graph replay)",
        "value": round(useful / (graph_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(graph_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"jagged_2k: {cfg.description}, N={cfg.max_seq_len}, "
                               f"seed {args.seed}", "outputs": "f32",
                   "total_tokens": w.total_tokens, "visible_pairs_all_heads": pairs},
        "eager_ms_per_step": round(eager_ms, 4),
        "eager_tflops": round(useful / (eager_ms * 1e-3) / 1e12, 2),
        "graph_ms_per_step": round(graph_ms, 4),
        "tokens_per_s": round(w.total_tokens / (graph_ms * 1e-3), 1),
        "roofline": {"kernel": "step (fwd + bwd), compulsory bytes", "bound": "hbm",
                     "achieved": round(hbm_gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(hbm_gbs / 8000.0, 4), "traffic": None,
                     "compulsory_bytes": int(compulsory)},
    }
    print(json.dumps(line), flush=True)


def bench_stu_layer(args):
    """One STU layer (the first, full-length layer of the 18-layer stack:
    B = 8, lengths U[2048, 4096], 64 targets, contextual 16, D = 512, H = 4,
    d = 128, K1 = 512, K2 = 64, N = 4096), forward with the attention output
    kept, then the backward with every parameter gradient.  Useful FLOPs: the
    two projections forward (2 T D NW + 2 T NU D) and backward (twice that:
    input and weight gradients), the attention's visible pairs (512 flop per
    pair and head forward, 1280 backward); the backward's recomputation of
    the projection is not counted."""
    import torch
    import sparse_sequence_attention_amd as sla
    from synthetic import make_stack_workload

    sw = make_stack_workload(seed=args.seed, layers=1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(args.seed + 1)
    T, D, H, d = int(sw.offsets[-1]), sw.hidden, sw.heads, sw.d
    NU, NW = H * d, 4 * H * d
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).bfloat16()  # noqa
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa
    x = bf(sw.x)
    dout = bf(rng.standard_normal((T, D), dtype=np.float32))
    ln1_w, ln2_w = f32(sw.ln1_w[0]), f32(sw.ln2_w[0])
    w_uvqk, w_out = bf(sw.w_uvqk[0]), bf(sw.w_out[0])
    offs = torch.from_numpy(sw.offsets).to(dev)
    tg = torch.from_numpy(sw.num_targets).to(dev)
    kw = dict(heads=H, d_qk=d, d_v=d, k1=sw.k1, k2=sw.k2, contextual_len=sw.contextual_len,
              max_seq_len=sw.max_seq_len)
    out = torch.empty_like(x)
    ws_f, ws_b = (torch.empty(sla.stu_layer_workspace_bytes(T, D, offs, tg, backward=b, **kw),
                              dtype=torch.uint8, device=dev) for b in (False, True))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        _, attn = sla.stu_layer_fwd(x, offs, tg, ln1_w, w_uvqk, ln2_w, w_out, out=out,
                                    want_attn=True, workspace=ws_f, **kw)
        if ev is not None:
            ev[1].record()
        g = sla.stu_layer_bwd(x, dout, offs, tg, ln1_w, w_uvqk, ln2_w, w_out, attn=attn,
                              workspace=ws_b, **kw)
        if ev is not None:
            ev[2].record()
        return g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    ms = fwd + bwd
    pairs = sla.count_pairs_host(sw.offsets, sw.num_targets, sw.k1, sw.k2, sw.contextual_len) * H
    gemm_fwd = 2 * T * D * NW + 2 * T * NU * D
    useful_fwd = gemm_fwd + pairs * 4 * d
    useful_bwd = 2 * gemm_fwd + pairs * 10 * d
    value = (useful_fwd + useful_bwd) / (ms * 1e-3) / 1e12
    line = {
        "metric": "STU layer fwd+bwd useful TFLOP/s (18-layer stack shape, full-length layer)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"stu_layer: B=8, L_b ~ U[2048, 4096], 64 targets, ctx 16, D={D}, "
                        f"H={H}, d={d}, K1={sw.k1}, K2={sw.k2}, N={sw.max_seq_len}, "
                        f"seed {args.seed}",
            "total_tokens": T,
            "visible_pairs_all_heads": pairs,
            "useful_flop_fwd": useful_fwd,
            "useful_flop_bwd": useful_bwd,
        },
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "phase_ms": {"fwd": round(fwd, 4), "bwd": round(bwd, 4)},
        "phase_tflops": {"fwd": round(useful_fwd / (fwd * 1e-3) / 1e12, 2),
                         "bwd": round(useful_bwd / (bwd * 1e-3) / 1e12, 2)},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


def bench_stu_stack(args):
    """The 18-layer STU stack forward (B = 8, L_b ~ U[2048, 4096], 64 targets,
    contextual 16, hidden 512, H = 4, d = 128, K1 = 512, K2 = 64, N = 4096;
    attention truncation before layer 9 keeps contextual 16 + the last 1024
    history tokens + the targets), random Xavier-uniform weights, bf16 or (with
    --fp8) FP8 projections.  A step is the whole stack, truncation included.
    Useful FLOPs per layer: 2 T_l D NW + 2 T_l NU D for the projections and
    512 per visible (row, key) pair and head for the attention."""
    import torch
    import sparse_sequence_attention_amd as sla
    from sparse_sequence_attention_amd.config import STUConfig
    from sparse_sequence_attention_amd.stack import STULayerWeights, stu_stack_fwd
    from synthetic import make_stack_workload

    sw = make_stack_workload(seed=args.seed)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = STUConfig(embedding_dim=sw.hidden, num_heads=sw.heads, hidden_dim=sw.d,
                    attention_dim=sw.d, sla_k1=sw.k1, sla_k2=sw.k2,
                    contextual_seq_len=sw.contextual_len, attn_num_layers=sw.layers,
                    attn_truncation_split_layer=sw.split_layer,
                    attn_truncation_tail_len=sw.tail_len, max_seq_len=sw.max_seq_len)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    layers = [STULayerWeights(ln1_w=f(sw.ln1_w[i]), w_uvqk=f(sw.w_uvqk[i]).bfloat16(),
                              ln2_w=f(sw.ln2_w[i]), w_out=f(sw.w_out[i]).bfloat16())
              for i in range(sw.layers)]
    if args.fp8:
        for w in layers:
            w.quantize_fp8()
    x = f(sw.x).bfloat16()
    offs = torch.from_numpy(sw.offsets).to(dev)
    tg = torch.from_numpy(sw.num_targets).to(dev)

    lens_host = np.diff(sw.offsets)

    def step():
        return stu_stack_fwd(cfg, layers, x, offs, tg, fp8=args.fp8, lengths_host=lens_host,
                             num_targets_host=sw.num_targets)

    for _ in range(args.warmup):
        res = step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        res = step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    H, d, D = sw.heads, sw.d, sw.hidden
    NU, NW = H * d, 4 * H * d
    full_pairs = sla.count_pairs_host(sw.offsets, sw.num_targets, sw.k1, sw.k2,
                                      sw.contextual_len) * H
    t_offs = res.offsets.cpu().numpy()
    t_tg = res.num_targets.cpu().numpy() if res.num_targets is not None else None
    trunc_pairs = sla.count_pairs_host(t_offs, t_tg, sw.k1, sw.k2, sw.contextual_len) * H
    useful = 0
    for li, T_l in enumerate(res.layer_tokens):
        pairs = full_pairs if li < sw.split_layer else trunc_pairs
        useful += 2 * T_l * D * NW + 2 * T_l * NU * D + pairs * 4 * d
    value = useful / (ms * 1e-3) / 1e12
    line = {
        "metric": "STU stack forward useful TFLOP/s (18 layers, truncation after layer 9)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"stu_stack: 18 layers, B=8, L_b ~ U[2048, 4096] (T={sw.offsets[-1]}), "
                        f"64 targets, ctx 16, D={D}, H={H}, d={d}, K1={sw.k1}, K2={sw.k2}, "
                        f"N={sw.max_seq_len}, truncation before layer {sw.split_layer} to "
                        f"ctx + {sw.tail_len} + targets, "
                        f"{'FP8' if args.fp8 else 'bf16'} projections, seed {args.seed}",
            "layer_tokens": res.layer_tokens,
            "useful_flop_per_step": useful,
        },
        "tokens_per_s": round(int(sw.offsets[-1]) / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


def bench_targets_fwd(args):
    """The target-aware SLA forward at inference (targets_16k: B = 16, each
    sequence a 16-token contextual prefix + U[8192, 16384] history tokens +
    256 candidate targets; K1 = 1024, K2 = 128, H = 4, d = 128, bf16 inputs
    and output).  A candidate sees the prefix, the history under the K1 / K2
    window of the first target slot, and itself.  A step is one sla_fwd call
    (schedule included); useful flops are 4d per visible pair and head."""
    import torch
    import sparse_sequence_attention_amd as sla
    from synthetic import make_sla_workload

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = make_sla_workload("targets_16k", seed=args.seed)
    t = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)  # noqa: E731
    q, k, v = t(w.q), t(w.k), t(w.v)
    offs = torch.from_numpy(w.offsets).to(dev)
    tg = torch.from_numpy(w.num_targets).to(dev)
    T, H, d = q.shape
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len,
              alpha=w.alpha)
    p = sla.make_problem(torch.bfloat16, offs, tg, T, H, d, d, w.k1, w.k2, w.contextual_len,
                         w.max_seq_len, w.alpha)
    ws = torch.empty(max(1, sla.workspace_size(p, sla.SLA_OP_FWD)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(q)

    def step():
        sla.sla_fwd(q, k, v, offs, tg, out=out, workspace=ws, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    pairs = sla.count_pairs_host(w.offsets, w.num_targets, w.k1, w.k2, w.contextual_len) * H
    useful = pairs * 4 * d
    value = useful / (ms * 1e-3) / 1e12
    line = {
        "metric": "target-aware SLA forward useful TFLOP/s and tokens/s at L=16K (inference)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"targets_16k: B=16, 16 ctx + U[8192,16384] history + 256 targets per "
                        f"sequence (T={T}), K1={w.k1}, K2={w.k2}, H={H}, d={d}, "
                        f"N={w.max_seq_len}, bf16 in and out, seed {args.seed}",
            "visible_pairs_all_heads": pairs,
            "useful_flop_per_step": useful,
        },
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "roofline": {"kernel": "fwd", "bound": "mfma", "achieved": round(value, 2),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_MFMA_TFLOPS, 4), "traffic": None},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


def bench_mfalcon(args):
    """Candidate scoring against a cached history (M-FALCON): the targets_16k
    histories (B = 16, 16 contextual + U[8192, 16384] tokens; K1 = 1024,
    K2 = 128, H = 4, d = 128, N = 16656) with their keys/values resident, and
    `--candidates` candidates per sequence scored in microbatches of
    `--microbatch` per sequence (one sla_fwd_candidates call each).  A step
    scores every candidate once.  Useful FLOPs: 4d per (candidate, visible
    key, head); each candidate sees the history window of the first
    candidate slot, the global prefix below it, and itself."""
    import torch
    import sparse_sequence_attention_amd as sla
    from synthetic import CONFIGS

    cfg = CONFIGS["targets_16k"]
    rng = np.random.default_rng(args.seed)
    hist = [L - 256 for L in cfg.lengths(rng)]  # the sequences without their 256 targets
    B, H, d = len(hist), cfg.heads, cfg.d
    m, bm = args.candidates, min(args.microbatch, args.candidates)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ho = np.concatenate([[0], np.cumsum(hist)]).astype(np.int64)
    Th = int(ho[-1])

    def normal(n):
        x = torch.empty((n, H, d), dtype=torch.float32, device=dev)
        x.normal_(0.0, cfg.std, generator=torch.Generator(device=dev).manual_seed(n + args.seed))
        return x.bfloat16()

    kh, vh = normal(Th), normal(Th + 1)[:Th].contiguous()
    C = B * m
    qc, kc, vc = normal(C), normal(C + 2)[:C].contiguous(), normal(C + 3)[:C].contiguous()
    out = torch.empty_like(qc)
    hist_offs = torch.from_numpy(ho).to(dev)
    kw = dict(k1=cfg.k1, k2=cfg.k2, contextual_len=cfg.contextual_len,
              max_seq_len=cfg.max_seq_len)
    # microbatch j: candidates [j*bm, (j+1)*bm) of every sequence, as views
    # of one [B][m] candidate layout
    nmb = (m + bm - 1) // bm
    views = []
    for j in range(nmb):
        n = min(bm, m - j * bm)
        idx = (torch.arange(B, device=dev)[:, None] * m + j * bm +
               torch.arange(n, device=dev)[None, :]).reshape(-1)
        offs = torch.arange(0, B * n + 1, n, dtype=torch.int64, device=dev)
        views.append((offs, qc[idx].contiguous(), kc[idx].contiguous(), vc[idx].contiguous(),
                      torch.empty((B * n, H, d), dtype=torch.bfloat16, device=dev)))
    ws = torch.empty(max(1, sla.workspace_size(sla.make_problem(torch.bfloat16, hist_offs, None,
                                                                max(Th, B * bm), H, d, d,
                                                                cfg.k1, cfg.k2,
                                                                cfg.contextual_len,
                                                                cfg.max_seq_len),
                                               sla.SLA_OP_FWD)),
                     dtype=torch.uint8, device=dev)

    def step():
        for offs, q_, k_, v_, o_ in views:
            sla.sla_fwd_candidates(kh, vh, hist_offs, q_, k_, v_, offs, out=o_, workspace=ws,
                                   **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    K2e = max(cfg.k2, cfg.contextual_len)
    per_cand = 0
    for U in hist:
        w0 = max(0, U - cfg.k1 + 1)
        per_cand += (U - w0) + min(K2e, w0, U) + 1
    pairs = per_cand * m * H
    useful = pairs * 4 * d
    value = useful / (ms * 1e-3) / 1e12
    line = {
        "metric": "M-FALCON candidate scoring useful TFLOP/s and candidates/s (cached history)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"mfalcon: B={B} histories of 16 ctx + U[8192,16384] tokens "
                        f"(T_hist={Th}), {m} candidates per sequence in microbatches of {bm}, "
                        f"K1={cfg.k1}, K2={cfg.k2}, H={H}, d={d}, N={cfg.max_seq_len}, "
                        f"seed {args.seed}",
            "candidates_per_step": B * m,
            "calls_per_step": nmb,
            "visible_pairs_all_heads": pairs,
            "useful_flop_per_step": useful,
        },
        "candidates_per_s": round(B * m / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, sample_tokens):
    """The fp64 oracle as it stands, on a bounded sample: the first whole
    sequences of the same workload (all heads) up to about `sample_tokens`
    tokens, forward + backward."""
    import oracle
    import sparse_sequence_attention_amd as sla
    ends = np.asarray(w.offsets[1:])
    reach = np.nonzero(ends >= sample_tokens)[0]
    m = int(reach[0]) + 1 if len(reach) else len(ends)  # sequences in the sample
    n = int(ends[m - 1])
    offs = np.asarray(w.offsets[:m + 1], np.int64)
    q, k, v, do = w.q[:n], w.k[:n], w.v[:n], w.dout[:n]
    t0 = time.perf_counter()
    oracle.sla_fwd(q, k, v, offs, None, w.k1, w.k2, w.contextual_len, w.max_seq_len)
    oracle.sla_bwd(q, k, v, do, offs, None, w.k1, w.k2, w.contextual_len, w.max_seq_len)
    t = time.perf_counter() - t0
    H, d = q.shape[1], q.shape[2]
    pairs = sla.count_pairs_host(offs, None, w.k1, w.k2, w.contextual_len) * H
    useful = pairs * (2 * (d + d) + 2 * (3 * d + 2 * d))
    return {"value": round(useful / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"sequences 0-{m - 1} of the workload ({n} tokens, lengths "
                      f"{[int(x) for x in np.diff(offs)]}), all {H} heads, fwd+bwd "
                      f"({t:.2f} s; {n / t:.1f} tokens/s)"}


if __name__ == "__main__":
    main()
