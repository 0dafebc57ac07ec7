"""Benchmark of the FP4 routed-expert MoE layer on one MI355X.

One step = the whole layer on one batch of synthetic inputs already resident
in HBM, as one library call (moe_fp4_layer_forward: routing, sort/permute,
MXFP8 of x, gate/up GEMM + SwiGLU, down GEMM, combine), on one stream.
The default workload is the largest one, the prefill layer with Zipf-skewed
routing (T=16384, H=7168, I=2048, E=256, top-8); after it the same process
times the pages' prompt-length prefill (T=4604, reported as prefill_leg) and
the decode layer (T=8, H=4096, I=1536, E=64, top-6, reported as decode_leg).
Copies of the packed weights are cycled where one step's weights would fit
the 256 MB Infinity Cache, so that it cannot serve them from the step before.

Prints ONE JSON line (rank 0).  The dominant kernel (the gate/up expert GEMM)
is timed with HIP events on the stream it runs on, bracketing each of its
launches in K further steps of the same layer run stage by stage through the
single-stage calls right after the timed steps (same inputs, same weight
copies); its algorithmic bytes (decode) or flops (prefill) per launch give
the roofline fraction against 8 TB/s or the dense FP8 MFMA peak.  The CPU baseline is the
oracle (plain C, fp32 accumulation) on the host's cores, on a bounded sample
of the same workload.

With --full a step starts from x alone (moe_fp4_layer_forward_full): the router
logits come from a bf16 GEMM and --n-shared shared experts, packed after the
routed ones, join every token's slots; the router's HIP-event time (the
stand-alone call, GEMM plus slice sum) and its roofline against HBM are
reported beside the gate/up kernel's.

--config d1 / d3 measures the FP8 dense projection instead (one step = MXFP8
quantisation of x + moe_fp8_dense_forward), with its own roofline line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DENSE_DECODE_KERNEL = "dense_decode_kernel<16, 2, 2, true, 1>"   # the instantiations the library launches
DENSE_PREFILL_KERNEL = "dense_dma_kernel"  # (prefill at the d3 shape: the 256 x 256 LDS-DMA tiles)
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense FP8 (and FP8 x FP4 scaled MFMA at the FP8 issue rate)
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense FP4 x FP4 (reported beside: the mixed FP8 x FP4 MFMA issues at the FP8 rate)
METRIC = "MoE-layer tokens/s + achieved HBM TB/s (decode) / MFMA util (prefill), 1 GPU"


def weight_bytes_per_expert(H: int, I: int, mats: int) -> float:
    # packed e2m1 nibbles (1/2 B) + one E8M0 byte per 32 elements
    return mats * H * I * (0.5 + 1.0 / 32)


def rocprof_summary(paths) -> str:
    """Markdown summary of rocprofv3 CSV outputs (kernel stats and, if present,
    per-dispatch counters averaged per kernel)."""
    import csv
    import glob
    out = []
    files = []
    for p in paths:
        files += glob.glob(os.path.join(p, "**", "*.csv"), recursive=True) if os.path.isdir(p) else [p]
    for f in sorted(files):
        rows = list(csv.DictReader(open(f)))
        if not rows:
            continue
        if f.endswith("kernel_stats.csv"):
            out.append(f"### kernel stats ({os.path.basename(f)})\n")
            out.append("| kernel | calls | avg us | min us | max us | total ms | % |")
            out.append("|---|---|---|---|---|---|---|")
            for r in rows:
                name = r["Name"].replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "").split("(")[0]
                out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                           f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                           f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
            out.append("")
        elif f.endswith("counter_collection.csv"):
            agg = {}
            for r in rows:
                name = r["Kernel_Name"].replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "").split("(")[0]
                key = (name, r["Counter_Name"])
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
            out.append(f"### counters per dispatch ({os.path.basename(f)})\n")
            out.append("| kernel | counter | dispatches | mean per dispatch |")
            out.append("|---|---|---|---|")
            for (name, cn), v in sorted(agg.items()):
                out.append(f"| {name} | {cn} | {len(v)} | {np.mean(v):.1f} |")
            out.append("")
    return "\n".join(out)


KERNEL_SOURCES = {
    "up_decode_kernel<1>": "fp4_routed_expert_amd/csrc/expert_decode.hip",
    "prefill_gemm_kernel<true>": "fp4_routed_expert_amd/csrc/expert_prefill.hip",
    DENSE_DECODE_KERNEL: "fp4_routed_expert_amd/csrc/dense.hip",
    DENSE_PREFILL_KERNEL: "fp4_routed_expert_amd/csrc/dense.hip",
}


def source_sha256(kernel: str) -> str:
    import hashlib
    return hashlib.sha256(open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb").read()).hexdigest()


def _counter_means(path: str, counter: str):
    """Per-kernel list of per-dispatch values of one counter from a rocprofv3 CSV directory."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "").split("(")[0]
            name = name.replace("void ", "")
            out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_dir: str, write_dir: str, kernel: str, workload: str, cfg: str = "c1",
                    steps: int = 20) -> str:
    """HBM traffic per launch of `kernel` from a FETCH_SIZE run and a WRITE_SIZE run,
    each counter scaled so that the 1 GiB device copies of --copy-calibration
    read and write exactly 1 GiB."""
    f = _counter_means(fetch_dir, "FETCH_SIZE")
    w = _counter_means(write_dir, "WRITE_SIZE")
    copy = [k for k in f if "copyBuffer" in k]
    if not copy or kernel not in f or kernel not in w:
        raise SystemExit(f"missing kernels in counter runs: have {sorted(f)}")
    cf = sorted(f[copy[0]])[-20:]   # the calibration copies are the largest copy dispatches
    cw = sorted(w[copy[0]])[-20:]
    gib_kib = float(1 << 20)
    fetch_scale = gib_kib / (sum(cf) / len(cf))
    write_scale = gib_kib / (sum(cw) / len(cw))
    kf = sum(f[kernel]) / len(f[kernel])
    kw = sum(w[kernel]) / len(w[kernel])
    traffic = (kf * fetch_scale + kw * write_scale) * 1024.0
    lines = [
        f"# HBM traffic: {kernel}, {workload}",
        "",
        "Commands (repo root, one MI355X; each counter in its own run):",
        "",
        "```",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o f -- python3 bench.py "
        f"--config {cfg} --decode-leg '' --steps {steps} --warmup 2 --cpu-budget 0 --copy-calibration",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o w -- python3 bench.py "
        f"--config {cfg} --decode-leg '' --steps {steps} --warmup 2 --cpu-budget 0 --copy-calibration",
        f"python3 bench.py --traffic-summary {fetch_dir} {write_dir} --kernel '{kernel}' "
        f"--workload '{workload}' --config {cfg} --steps {steps}",
        "```",
        "",
        "The 1 GiB copies of --copy-calibration run in the same process; FETCH_SIZE reads half",
        "of the bytes a copy moves, so it is scaled by the factor below.",
        "",
        f"- dispatches: {len(f[kernel])} (FETCH_SIZE run), {len(w[kernel])} (WRITE_SIZE run)",
        f"- FETCH_SIZE per dispatch: {kf:.1f} KiB (raw)",
        f"- WRITE_SIZE per dispatch: {kw:.1f} KiB (raw)",
        f"- calibration: 1 GiB device copy reads as FETCH_SIZE {sum(cf) / len(cf):.1f} KiB, "
        f"WRITE_SIZE {sum(cw) / len(cw):.1f} KiB; scale factors {fetch_scale:.4f} / {write_scale:.4f}",
        f"- source_sha256: {source_sha256(kernel)}",
        f"- traffic_bytes_per_launch: {traffic:.0f}",
        "",
    ]
    return "\n".join(lines)


# MI355X: 8 XCDs (GRBM_GUI_ACTIVE sums one count per XCD), 256 CUs x 4 SIMDs.
N_XCD, N_SIMD = 8, 1024
MFMA_KERNELS = {  # kernel -> flops per launch as a function of the layer shape (P = T * k)
    "prefill_gemm_kernel<true>": lambda sh: 4.0 * sh.H * sh.I * sh.T * sh.k,
    "prefill_gemm_kernel<false>": lambda sh: 2.0 * sh.H * sh.I * sh.T * sh.k,
}


def mfma_summary(pmc_dir: str, workload: str, cfg: str, steps: int) -> str:
    """Clock and MFMA activity of the prefill GEMMs from one counter run
    (GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES, SQ_VALU_MFMA_BUSY_CYCLES): the SCLK the
    kernel ran at (active cycles per XCD over its duration), the share of SIMD
    cycles with the MFMA pipe busy, and the flop rate against the 5.0 PF FP8
    peak (at 2.4 GHz) and against that peak scaled to the measured clock."""
    import csv
    import glob
    import synth
    sh = synth.CONFIGS[cfg]
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "").split("(")[0]
            name = name.replace("void ", "")
            d = per.setdefault(name, {}).setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = [
        f"# MFMA activity and clock: prefill GEMMs, {workload}",
        "",
        "Commands (repo root, one MI355X; one counter run):",
        "",
        "```",
        f"rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES --output-format csv "
        f"-d {pmc_dir} -o m -- python3 bench.py --config {cfg} --decode-leg '' --steps {steps} --warmup 2 "
        f"--cpu-budget 0",
        f"python3 bench.py --mfma-summary {pmc_dir} --workload '{workload}' --config {cfg} --steps {steps}",
        "```",
        "",
        f"SCLK = GRBM_GUI_ACTIVE / {N_XCD} XCDs / kernel duration; MFMA busy = "
        f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} x {N_SIMD} SIMDs); flop rate = the "
        "algorithmic flops of one launch over its duration (durations are those of the counter run, "
        "where kernels run serialised).",
        "",
        "| kernel | dispatches | duration us | SCLK GHz | MFMA busy | PFLOP/s | of 5.0 PF | of the peak at that SCLK |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for kern, flops in MFMA_KERNELS.items():
        ds = [d for d in per.get(kern, {}).values()
              if all(c in d for c in ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES"))]
        if not ds:
            raise SystemExit(f"no dispatches of {kern} with the counters in {pmc_dir}: have {sorted(per)}")
        ns = float(np.mean([d["ns"] for d in ds]))
        cyc = float(np.mean([d["GRBM_GUI_ACTIVE"] for d in ds])) / N_XCD
        busy = float(np.mean([d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds])) / (cyc * N_SIMD)
        ghz = cyc / ns
        pf = flops(sh) / (ns * 1e-9) / 1e15
        lines.append(f"| {kern} | {len(ds)} | {ns / 1e3:.1f} | {ghz:.2f} | {100 * busy:.1f} % | {pf:.2f} | "
                     f"{100 * pf / 5.0:.1f} % | {100 * pf / (5.0 * ghz / 2.4):.1f} % |")
    lines.append("")
    return "\n".join(lines)


def load_traffic(kernel: str, workload: str):
    """traffic_bytes_per_launch from the committed summary, if it was taken on
    the kernel source as it is now (else None)."""
    import glob
    for f in glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md")):
        text = open(f).read()
        if f"# HBM traffic: {kernel}, {workload}" not in text:
            continue
        sha = traffic = None
        for line in text.splitlines():
            if line.startswith("- source_sha256: "):
                sha = line.split(": ", 1)[1].strip()
            if line.startswith("- traffic_bytes_per_launch: "):
                traffic = float(line.split(": ", 1)[1])
        if sha == source_sha256(kernel) and traffic is not None:
            return traffic
    return None


def copy_calibration(reps: int = 20):
    """A plain device copy of 1 GiB, `reps` times: 1 GiB read + 1 GiB written per
    dispatch, the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def oracle_threads() -> int:
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return min(threads, len(os.sched_getaffinity(0)))


def cpu_baseline(name: str, budget_s: float):
    """The oracle as it stands on a bounded sample of the workload: whole-layer
    rows (route, MXFP8 of x, the k expert FFNs, combine) of tokens drawn without
    replacement by a seeded generator, one token per call, until `budget_s` of
    wall time is spent (at least one token).  tokens/s = tokens done / time."""
    import oracle
    import synth
    inp = synth.make_inputs(name)
    T = inp.shape.T
    order = np.random.default_rng(12345).permutation(T).astype(np.int32)
    oracle.layer_tokens(inp, order[:1])  # warm the page cache of the weights
    n_tok = 0
    t0 = time.perf_counter()
    while n_tok == 0 or time.perf_counter() - t0 < budget_s:
        oracle.layer_tokens(inp, order[n_tok % T:n_tok % T + 1])
        n_tok += 1
    dt = time.perf_counter() - t0
    drawn = (f"{n_tok} of the {T} tokens of the {name} workload (seeded random draw)" if n_tok <= T else
             f"the {T} tokens of the {name} workload in seeded random order, cycled: {n_tok} token layers")
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"{drawn}, whole layer per token in {dt:.1f} s ({oracle.PRECISION} plain C, "
                      f"OpenMP over output rows)"}


def cpu_baseline_dense(name: str, budget_s: float):
    import oracle
    import synth
    inp = synth.make_dense_inputs(name)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    n_tok = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.dense_fp8(xq, xs, inp.wq, inp.ws, np.array([n_tok % inp.shape.T], dtype=np.int32))
        n_tok += 1
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"{n_tok} single-token rows of the {name} projection in {dt:.1f} s "
                      f"(fp64 plain C, OpenMP over the output rows; x quantised beforehand)"}


def bench_dense(args):
    """One step = moe_quant_act_mxfp8 + moe_fp8_dense_forward on one batch of rows."""
    import torch

    import fp4_routed_expert_amd as moe
    import synth

    dev = torch.device("cuda:0")
    inp = synth.make_dense_inputs(args.config)
    sh = inp.shape
    T, K, N = sh.T, sh.K, sh.N
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    wq, ws = t(inp.wq), t(inp.ws)
    nbytes = moe._lib.lib().moe_fp8_dense_packed_bytes(N, K)
    copies = args.copies or max(1, min(8, int(np.ceil(2.0e9 / nbytes))))
    dws = [moe.dense_prepack(wq, ws) for _ in range(copies)]
    del wq, ws
    x = t(inp.x.view(np.int16)).view(torch.bfloat16)
    xq = torch.empty((T, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, K // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i, timed=None):
        moe.quant_act_mxfp8(x, xq, xs)
        if timed is not None:
            ev[timed][0].record()
        moe.dense_forward(dws[i % copies], xq, xs, args.flags, y=y)
        if timed is not None:
            ev[timed][1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    decode = args.flags == 1 or (args.flags == 0 and T <= 96)
    b_alg = N * K * (1 + 1 / 32) + T * K * (1 + 1 / 32) + T * N * 2
    f_alg = 2.0 * T * N * K
    wl = synth.DENSE_NAMES.get(args.config, args.config)
    if decode:
        ach = b_alg / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": DENSE_DECODE_KERNEL + " (FP8 weight streaming)", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": load_traffic(DENSE_DECODE_KERNEL, wl),
                "alg_bytes_per_launch": b_alg, "avg_launch_us": k_ms * 1e3}
    else:
        ach = f_alg / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": DENSE_PREFILL_KERNEL + " (LDS-DMA FP8 GEMM, 256 x 256 tiles)", "achieved": ach,
                "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_FP8_PEAK_TFLOPS,
                "traffic": load_traffic(DENSE_PREFILL_KERNEL, wl),
                "alg_flops_per_launch": f_alg, "avg_launch_us": k_ms * 1e3}
    if args.copy_calibration:
        copy_calibration()
    ms = dt / args.steps * 1e3
    line = {
        "metric": "FP8 dense projection tokens/s + achieved HBM TB/s (decode) / MFMA util (prefill), 1 GPU",
        "value": T * args.steps / dt, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3xfp8e4m3->bf16", "data": "synthetic",
        "config": {"workload": synth.DENSE_NAMES.get(args.config, args.config), "T": T, "K": K, "N": N,
                   "seed": sh.seed, "weight_copies": copies, "path_flags": args.flags, "launch": "eager"},
        "roofline": roof,
        "cpu_baseline": cpu_baseline_dense(args.config, args.cpu_budget) if args.cpu_budget > 0 else None,
    }
    print(json.dumps(line), flush=True)


def bench_shard(args):
    """One GPU's share of the layer: EP (the gate/up and down calls over experts
    0..E/G-1 on the full routing's pairs) or TP (the whole layer call over the
    intermediate rows 0..I/G-1, a partial y)."""
    import torch

    import fp4_routed_expert_amd as moe
    import synth
    from fp4_routed_expert_amd import shard

    kind, G = args.shard.split(":")
    G = int(G)
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(args.config)
    sh = inp.shape
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    w = [t(getattr(inp, n)) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]
    x = t(inp.x.view(np.int16)).view(torch.bfloat16)
    logits = t(inp.logits)
    if kind == "ep":
        Eg = E // G
        cw = shard.ep_weights(*w, 0, Eg)
        Ig = I
    elif kind == "tp":
        Eg, Ig = E, I // G
        cw = shard.tp_slice(*w, 0, Ig)
    else:
        raise SystemExit(f"--shard {args.shard}: expected ep:G or tp:G")
    del w
    nbytes = moe.packed_weight_bytes(Eg, H, Ig)
    copies = args.copies or max(1, min(8, int(np.ceil(2.0e9 / nbytes))))
    pws = [moe.prepack_weights(*cw) for _ in range(copies)]
    del cw
    P = T * k
    ids, gates = moe.route_topk(logits, k)
    counts, offsets, sp, pp = moe.sort_permute(ids, E)
    xq, xs = moe.quant_act_mxfp8(x)
    if kind == "ep":
        o_g, sp_g, (r0, r1) = shard.ep_segment(offsets, sp, 0, Eg)
        used = int((counts[:Eg] > 0).sum())
        rows = r1 - r0
        hq = torch.empty((P, Ig), dtype=torch.uint8, device=dev)
        hs = torch.empty((P, Ig // 32), dtype=torch.uint8, device=dev)
        O = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
        sws = torch.empty(max(moe.stage_workspace_size(T, Eg, k, H, Ig), 256), dtype=torch.uint8, device=dev)

        def step(i):
            pw = pws[i % copies]
            moe.expert_up(pw, xq, xs, o_g, sp_g, T, k, args.flags, hq=hq, hs=hs, workspace=sws)
            moe.expert_down(pw, hq, hs, o_g, T, k, args.flags, O=O, workspace=sws)
    else:
        used = int((counts > 0).sum())
        rows = P
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        lws = torch.empty(max(moe.layer_workspace_size(T, Eg, k, H, Ig, args.flags), 256), dtype=torch.uint8,
                          device=dev)

        def step(i):
            moe.layer_forward(pws[i % copies], x, logits, k, args.flags, y=y, workspace=lws)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3
    b_w = used * weight_bytes_per_expert(H, Ig, 3)
    flops = 6.0 * H * Ig * rows
    name = synth.CONFIG_NAMES.get(args.config, args.config)
    what = (f"EP shard 1/{G} (experts 0..{Eg - 1}: gate/up + down over their {rows} pairs)" if kind == "ep"
            else f"TP shard 1/{G} (intermediate rows 0..{Ig - 1}: the whole layer, a partial y)")
    line = {
        "metric": METRIC, "value": T * args.steps / dt, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4e2m1xfp8e4m3->fp32", "data": "synthetic",
        "config": {"workload": f"{name}, {what}", "T": T, "H": H, "I_shard": Ig, "E_shard": Eg, "k": k,
                   "used_experts": used, "pairs": rows, "weight_copies": copies, "path_flags": args.flags},
        "shard_weight_tbps": b_w / (ms * 1e-3) / 1e12,
        "shard_hbm_frac": b_w / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "shard_mfma_frac_fp8": flops / (ms * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4",
                    help="workload name: c0-c4 the MoE layer (c4, the largest, is the headline), d0-d3 "
                         "the FP8 dense projection")
    ap.add_argument("--decode-leg", default="c1",
                    help="layer workload timed after the main one in the same process and reported "
                         "as decode_leg (the metric's HBM-bound part); '' = none")
    ap.add_argument("--prefill-leg", default="c3",
                    help="layer workload timed after the main one and reported as prefill_leg (the "
                         "metric's other MFMA-bound shape); runs only with a decode leg ('' = none)")
    ap.add_argument("--flags", type=int, default=0, help="1 = force decode path, 2 = force prefill path")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time; 0 = skip")
    ap.add_argument("--copies", type=int, default=0, help="weight copies cycled (0 = auto)")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the layer call (one graph per weight copy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 20 plain 1 GiB device copies (HBM counter calibration)")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="PATH",
                    help="print a markdown summary of rocprofv3 CSV outputs and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic summary of --kernel from two counter runs and exit")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="print the clock / MFMA-busy summary of the prefill GEMMs from a counter run and exit")
    ap.add_argument("--full", action="store_true",
                    help="step = router GEMM + layer + shared expert (moe_fp4_layer_forward_full)")
    ap.add_argument("--n-shared", type=int, default=1,
                    help="shared experts with --full (packed after the routed ones, same I)")
    ap.add_argument("--shard", default="",
                    help="ep:G or tp:G -- time one GPU's share of the layer (experts 0..E/G-1, or "
                         "the intermediate rows 0..I/G-1); the exchanges between GPUs are not run")
    ap.add_argument("--kernel", default="up_decode_kernel<1>")
    ap.add_argument("--workload", default="")
    args = ap.parse_args()
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary))
        return
    if args.mfma_summary:
        print(mfma_summary(args.mfma_summary, args.workload, args.config, args.steps))
        return
    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.kernel, args.workload,
                              args.config, args.steps))
        return
    if args.config.startswith("d"):
        if args.gpus != 1:
            print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
            sys.exit(2)
        bench_dense(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design note, not a measured path)", file=sys.stderr)
        sys.exit(2)
    if args.shard:
        bench_shard(args)
        return

    line = measure_layer(args, args.config, args.steps, args.warmup)
    if args.decode_leg and args.prefill_leg and args.config != args.prefill_leg and not args.shard:
        # the metric's other prefill shape (T4604, the pages' prompt length),
        # same process, after the main workload's memory is released
        import torch
        torch.cuda.empty_cache()
        p = measure_layer(args, args.prefill_leg, args.steps, args.warmup)
        line["prefill_leg"] = {
            "workload": p["config"]["workload"], "value": p["value"], "unit": p["unit"],
            "ms_per_step": p["ms_per_step"], "step_ms_p10_p50_p90": p["step_ms_p10_p50_p90"],
            "layer_mfma_frac_fp8": p["layer_mfma_frac_fp8"], "roofline": p["roofline"]}
    if args.decode_leg and args.config != args.decode_leg and not args.shard:
        # the decode-shaped leg of the metric (achieved HBM TB/s), same process,
        # after the prefill-shaped workload's memory is released
        import torch
        torch.cuda.empty_cache()
        d = measure_layer(args, args.decode_leg, args.steps, args.warmup)
        line["decode_leg"] = {
            "workload": d["config"]["workload"], "value": d["value"], "unit": d["unit"],
            "ms_per_step": d["ms_per_step"], "step_ms_p10_p50_p90": d["step_ms_p10_p50_p90"],
            "layer_hbm_tbps": d["layer_hbm_tbps"], "layer_hbm_frac": d["layer_hbm_frac"],
            "used_experts": d["config"]["used_experts"], "roofline": d["roofline"]}
    if args.copy_calibration:
        copy_calibration()
    line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget) if args.cpu_budget > 0 else None
    print(json.dumps(line), flush=True)


def measure_layer(args, cfg: str, steps: int, warmup: int) -> dict:
    """Time `steps` layer steps of workload `cfg` after `warmup` untimed ones;
    returns the JSON line's fields (cpu_baseline aside)."""
    import torch

    import fp4_routed_expert_amd as moe
    import synth

    dev = torch.device("cuda:0")
    inp = synth.make_inputs(cfg)
    sh = inp.shape
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    # --full: ns shared experts packed after the E routed ones, every token's
    # slots = k routed + ns shared
    ns = max(args.n_shared, 0) if args.full else 0
    Ew, kk = E + ns, k + ns
    P = T * kk
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    sws = [synth.make_shared_weights(dataclasses.replace(sh, seed=sh.seed + 1000 * i)) for i in range(ns)]
    canon = [t(np.concatenate([getattr(inp, n)] + [sw[j] for sw in sws], axis=0)) for j, n in enumerate(names)]
    del sws
    packed_bytes = moe.packed_weight_bytes(Ew, H, I)
    copies = args.copies or max(1, min(8, int(np.ceil(2.0e9 / packed_bytes))))
    pws = [moe.prepack_weights(*canon) for _ in range(copies)]
    del canon
    x = t(inp.x.view(np.int16)).view(torch.bfloat16)
    logits = t(inp.logits)
    del inp
    if args.full:
        # router weights, one copy per weight copy
        wg = [t(synth.make_router_weights(sh).view(np.int16)).view(torch.bfloat16) for _ in range(copies)]
        r_ws = torch.empty(max(moe.router_workspace_size(T, H, E), 256), dtype=torch.uint8, device=dev)

    # all outputs and workspaces allocated once, outside the timed region
    ids = torch.empty((T, kk), dtype=torch.int32, device=dev)
    gates = torch.empty((T, kk), dtype=torch.float32, device=dev)
    ids[:, k:] = torch.arange(E, Ew, dtype=torch.int32, device=dev)
    gates[:, k:] = 1.0
    ids_r = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates_r = torch.empty((T, k), dtype=torch.float32, device=dev)
    sort_out = (torch.empty(Ew, dtype=torch.int32, device=dev), torch.empty(Ew + 1, dtype=torch.int32, device=dev),
                torch.empty(P, dtype=torch.int32, device=dev), torch.empty(P, dtype=torch.int32, device=dev))
    from fp4_routed_expert_amd import _lib
    sort_ws_n = _lib.lib().moe_sort_permute_workspace_size(T, Ew, kk)
    sort_ws = torch.empty(max(sort_ws_n, 256), dtype=torch.uint8, device=dev)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    hq = torch.empty((P, I), dtype=torch.uint8, device=dev)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=dev)
    O = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    stage_ws = torch.empty(max(_lib.lib().moe_fp4_stage_workspace_size(T, Ew, kk, H, I), 256),
                           dtype=torch.uint8, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    ev_r = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)]
    if args.full:
        lws = torch.empty(max(moe.layer_full_workspace_size(T, Ew, k, H, I, ns, args.flags), 256),
                          dtype=torch.uint8, device=dev)
    else:
        lws = torch.empty(max(moe.layer_workspace_size(T, E, k, H, I, args.flags), 256),
                          dtype=torch.uint8, device=dev)

    def step(i):
        if args.full:
            moe.layer_forward_full(pws[i % copies], ns, wg[i % copies], x, k, args.flags, y=y,
                                   workspace=lws)
        else:
            moe.layer_forward(pws[i % copies], x, logits, k, args.flags, y=y, workspace=lws)

    def staged_step(i, timed_idx):
        pw = pws[i % copies]
        if args.full:
            ev_r[timed_idx][0].record()
            moe.router_logits(x, wg[i % copies], logits, workspace=r_ws)
            ev_r[timed_idx][1].record()
            moe.route_topk(logits, k, ids_r, gates_r)
            ids[:, :k] = ids_r
            gates[:, :k] = gates_r
        else:
            moe.route_topk(logits, k, ids, gates)
        counts, offsets, sp, pp = moe.sort_permute(ids, Ew, out=sort_out, workspace=sort_ws)
        moe.quant_act_mxfp8(x, xq, xs)
        ev[timed_idx][0].record()
        moe.expert_up(pw, xq, xs, offsets, sp, T, kk, args.flags, hq=hq, hs=hs, workspace=stage_ws)
        ev[timed_idx][1].record()
        moe.expert_down(pw, hq, hs, offsets, T, kk, args.flags, O=O, workspace=stage_ws)
        moe.combine(O, gates, pp, T, kk, H, y=y)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        # the layer call only enqueues kernels on the current stream (no allocation,
        # memset or host readback), so one call per weight copy is captured and replayed
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()

        def step(i):  # noqa: F811
            graphs[i % copies].replay()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dt = t1 - t0
    for i in range(steps):
        staged_step(warmup + i, i)
    torch.cuda.synchronize()
    up_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the spread of single steps: each layer call bracketed by its own events
    # (a separate loop, outside the timed region)
    for i in range(steps):
        ev[i][0].record()
        step(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    counts = sort_out[0].cpu().numpy()
    used = int((counts > 0).sum())

    ms_per_step = dt / steps * 1e3
    tokens_per_s = T * steps / dt
    # algorithmic bytes: weights of the experts that tokens were routed to, plus activations
    b_layer = used * weight_bytes_per_expert(H, I, 3) + T * H * 2 + T * E * 4 + T * H * 4
    b_up = used * weight_bytes_per_expert(H, I, 2) + T * H * (1 + 1 / 32) + P * I * (1 + 1 / 32)
    up_gbs = b_up / (up_ms * 1e-3) / 1e9
    flops = 6.0 * H * I * P
    up_flops = 4.0 * H * I * P
    prefill = args.flags == 2 or (args.flags == 0 and P > 16 * Ew)
    wl = synth.CONFIG_NAMES.get(cfg, cfg)
    if prefill:
        achieved = up_flops / (up_ms * 1e-3) / 1e12
        kname = "prefill_gemm_kernel<true>"
        roof = {"bound": "mfma", "kernel": kname + " (gate/up GEMM + SwiGLU + MXFP8 of h)",
                "achieved": achieved, "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_FP8_PEAK_TFLOPS,
                "frac_of_fp4_peak": achieved / MFMA_FP4_PEAK_TFLOPS,
                "traffic": load_traffic(kname, wl),
                "alg_flops_per_launch": up_flops, "avg_launch_us": up_ms * 1e3}
    else:
        kname = "up_decode_kernel<1>"
        roof = {"bound": "hbm", "kernel": kname + " (gate/up GEMM + SwiGLU + MXFP8 of h)",
                "achieved": up_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": up_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic(kname, wl),
                "alg_bytes_per_launch": b_up, "avg_launch_us": up_ms * 1e3}
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1xfp8e4m3->fp32",
        "data": "synthetic",
        "config": {"workload": wl, "T": T, "H": H, "I": I,
                   "E": E, "k": k, "seed": sh.seed, "used_experts": used, "weight_copies": copies,
                   "path_flags": args.flags, "launch": "hip_graph" if args.graph else "eager"},
        "step_ms_p10_p50_p90": [float(v) for v in np.percentile(step_ms, [10, 50, 90])],
        "layer_hbm_tbps": b_layer / (ms_per_step * 1e-3) / 1e12,
        "layer_hbm_frac": b_layer / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac_fp8": flops / (ms_per_step * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
        "roofline": roof,
    }
    if args.full:
        # router GEMM: bf16 x and Wg read once, fp32 logits written
        r_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_r]))
        r_bytes = T * H * 2 + E * H * 2 + T * E * 4
        r_gbs = r_bytes / (r_ms * 1e-3) / 1e9
        line["config"]["workload"] += f" + router GEMM + {ns} shared expert(s)"
        line["config"]["n_shared"] = ns
        r_kernel = ("router_dma_kernel" if T >= 128 and E >= 256 else
                    "router_tiled_kernel" if T >= 128 or (T > 16 and E >= 256) else "router_partial_kernel")
        r_tflops = 2.0 * T * H * E / (r_ms * 1e-3) / 1e12
        line["router"] = {"bound": "hbm", "kernel": f"{r_kernel} + slice sum (bf16 x . Wg, fp32 logits)",
                          "achieved": r_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": r_gbs / HBM_PEAK_GBS, "alg_bytes_per_launch": r_bytes,
                          "alg_flops_per_launch": 2.0 * T * H * E, "avg_launch_us": r_ms * 1e3,
                          "tflops": r_tflops, "frac_of_bf16_peak": r_tflops / MFMA_BF16_PEAK_TFLOPS}
        line["layer_hbm_tbps"] = (b_layer + E * H * 2) / (ms_per_step * 1e-3) / 1e12
        line["layer_hbm_frac"] = line["layer_hbm_tbps"] * 1e3 / HBM_PEAK_GBS
    return line


if __name__ == "__main__":
    main()
