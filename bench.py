#!/usr/bin/env python3
"""Benchmark of the Beam MoE block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode,prefill]
                    [--no-cpu-baseline]

A step is one beam_moe_forward call over one batch of synthetic input (router,
selection, dispatch, gate/up + SwiGLU, down, combine), inputs resident in HBM.
W untimed steps, then K timed steps between a synchronize and HIP events on
the launch stream.  The library's own stage events (beam_moe_timing_*) give
each kernel's average duration inside the same timed region, which feeds the
roofline figure of the dominant kernel.

Prints one JSON line.  Its headline is the decode batch (T=64, HBM-bound);
the prefill batch (T=16384, MFMA-bound) is reported in the same line under
"prefill" with its own roofline.

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
this script (FETCH_SIZE, then WRITE_SIZE) with --copy-calibration, which adds
one plain elementwise copy of known size whose counter readings give the
scale factors.  `python bench.py --summarize-pmc FETCH_DIR WRITE_DIR` turns
the two runs into the traffic file under profiles/; the roofline reports it
only while the expert kernel sources still hash to what was measured.
"""
from __future__ import annotations

import argparse
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import hashlib

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, published
METRIC = "MoE-layer tokens/s (decode T=64, prefill T=16K); % HBM BW / bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_hbm_traffic_decode_prefill.txt")
# sources whose code (comments aside) decides the expert kernels' memory traffic:
# the kernels, the launch plan and the tile table the dispatch writes
KERNEL_SOURCES = ["grouped_top_routing_fp32_amd/csrc/" + f
                  for f in ("common.h", "experts.hip", "grouped_gemm.hip", "dispatch.hip", "abi.cpp")]
COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read, 1 GiB written
# Workloads of the counter runs behind TRAFFIC_FILE: one per gate/up kernel.
TRAFFIC_WORKLOADS = "decode,prefill,decode_fp8,prefill_fp8"
# Workloads of the kernel-trace run behind the kernel-time profile.
TRACE_WORKLOADS = "decode,prefill,prefill_packed,decode_fp8,prefill_fp8"
GATE_UP_KERNELS = {"decode": "gateup_stream_lds_kernel", "prefill": "grouped_gemm_kernel<true, false",
                   "decode_fp8": "gateup_stream_fp8_kernel", "prefill_fp8": "grouped_gemm_kernel<true, true"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads",
                    default="decode,prefill,prefill_packed,decode_fp8,prefill_fp8,skewed,router_dispatch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-residual", action="store_true",
                    help="skip timing the residual-sublayer entry point on the same batches")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic file from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_MD"),
                    help="write a per-workload kernel time table from a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the decode/prefill line: tokens/s and roofline fractions over batch sizes T")
    ap.add_argument("--sweep-fp8", action="store_true", help="the T sweep through the FP8-weight entry point")
    ap.add_argument("--sweep-tokens", default="1,2,4,8,16,32,64,128,256,512,1024,2048,4096,8192,16384")
    ap.add_argument("--summarize-counters", nargs="+", metavar="OUT_MD WORKLOADS=COUNTER_DIR",
                    help="per-kernel counter summary of rocprofv3 --pmc runs of this script, one run per "
                         "WORKLOADS (the --workloads value it was given) and COUNTER_DIR")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="time the GEMM library on the prefill MoE shapes (context for the grouped GEMMs) and exit")
    ap.add_argument("--summarize-sweep", nargs=2, metavar=("SWEEP_JSON", "OUT_MD"),
                    help="write a markdown table from a --sweep JSON line and exit")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of KERNEL_SOURCES with comments and whitespace removed."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_counter_csv(d, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc csv run: [(kernel, value)]."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            per = {}
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = r["Dispatch_Id"]
                name, val = per.get(key, (r["Kernel_Name"], 0.0))
                per[key] = (name, val + float(r["Counter_Value"]))
            rows += [per[k] for k in sorted(per, key=int)]
    return rows


def summarize_pmc(fetch_dir, write_dir):
    fetch = read_counter_csv(fetch_dir, "FETCH_SIZE")
    write = read_counter_csv(write_dir, "WRITE_SIZE")

    def copy_kib(rows):
        vals = [v for n, v in rows if "neg" in n.lower()]
        if not vals:
            raise SystemExit("no calibration copy kernel in the counter run (was --copy-calibration given?)")
        return sum(vals) / len(vals)

    f_scale = COPY_BYTES / 1024.0 / copy_kib(fetch)
    w_scale = COPY_BYTES / 1024.0 / copy_kib(write)
    lines = ["# HBM traffic per launch of the gate/up kernel (decode and prefill, bf16 and FP8 weights), from rocprofv3 counters",
             "# fetch:  rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'beam::|neg' --output-format csv "
             "-d <FETCH_DIR> -o run -- "
             f"python3 bench.py --workloads {TRAFFIC_WORKLOADS} --steps 3 --warmup 1 --no-cpu-baseline --no-residual "
             "--copy-calibration",
             "# write:  rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'beam::|neg' --output-format csv "
             "-d <WRITE_DIR> -o run -- "
             f"python3 bench.py --workloads {TRAFFIC_WORKLOADS} --steps 3 --warmup 1 --no-cpu-baseline --no-residual "
             "--copy-calibration",
             "# (one workload per gate/up kernel: dispatches are told apart by kernel name)",
             "# summary: python3 bench.py --summarize-pmc <FETCH_DIR> <WRITE_DIR>",
             f"# calibration: elementwise copy (torch.neg) of {COPY_BYTES} bytes read and written;"
             f" FETCH_SIZE reads {copy_kib(fetch):.0f} KiB (scale {f_scale:.4f}),"
             f" WRITE_SIZE reads {copy_kib(write):.0f} KiB (scale {w_scale:.4f})",
             f"# expert kernel sources sha256[:16] = {kernel_source_hash()}"]
    for wl, pat in GATE_UP_KERNELS.items():
        fv = [v for n, v in fetch if pat in n]
        wv = [v for n, v in write if pat in n]
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        traffic = (fk * f_scale + wk * w_scale) * 1024.0
        lines.append(f"workload={wl} kernel={pat} dispatches={len(fv)} fetch_kib={fk:.0f} write_kib={wk:.0f} "
                     f"traffic_bytes={traffic:.0f} source_sha={kernel_source_hash()}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sweep(sweep_json, out_md):
    """Markdown table of a `bench.py --sweep` JSON line."""
    with open(sweep_json) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    fp8 = d["config"].get("weights", "bf16") != "bf16"
    out = ["# T sweep: Beam MoE block forward" + (" with FP8 E4M3 expert weights" if fp8 else "") +
           ", batch sizes 1 .. 16384 on one MI355X", "",
           "Command (repository root on the GPU host):", "", "```",
           "python3 bench.py --sweep" + (" --sweep-fp8" if fp8 else "") + " --steps 20 --warmup 3 > <SWEEP_JSON>",
           "python3 bench.py --summarize-sweep <SWEEP_JSON> <this file>", "```", "",
           "Per point: mean ms per forward step over the timed steps (fewer steps for large T), the",
           "expert path the library chose, and the layer's fraction of the HBM roofline (bytes of the",
           "touched experts' weights, router, x and out over the step time, against 8 TB/s) and of",
           "the bf16 MFMA roofline (expert FLOPs over the step time, against 2.5 PFLOP/s).", "",
           "| T | ms / step | tokens/s | path | experts touched | HBM fraction | MFMA fraction | gate/up ms | down ms |",
           "|---|---|---|---|---|---|---|---|---|"]
    for p in d["points"]:
        out.append(f"| {p['T']} | {p['ms_per_step']:.3f} | {p['tokens_per_s']:,.0f} | {p['path']} | "
                   f"{p['experts_touched']} | {p['layer_hbm_frac']:.3f} | {p['layer_mfma_frac']:.3f} | "
                   f"{p['stage_ms']['gate_up']:.3f} | {p['stage_ms']['down']:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_trace(trace_dir, out_md):
    """Per-workload kernel durations of the library's kernels from a kernel-trace run of this script.

    Calls are cut before each router_logits_kernel dispatch, or before the prenorm_kernel that
    opens a residual-sublayer call.  A call that ran the grouped GEMM is prefill, one that ran
    the FP8 kernels decode_fp8, the others decode; residual-sublayer calls (prenorm present)
    get a section of their own."""
    import csv
    import glob
    path = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))[0]
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if "beam::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    calls, cur = [], []
    for r in rows:
        name = r["Kernel_Name"]
        opens = "prenorm_kernel" in name or (
            "router_logits_kernel" in name and not (cur and "prenorm_kernel" in cur[-1]["Kernel_Name"]))
        if opens and cur:
            calls.append(cur)
            cur = []
        cur.append(r)
    if cur:
        calls.append(cur)

    def short(name):
        name = name.replace("void ", "")
        return name[:name.index("(")] if "(" in name else name

    def kind(c):
        names = " ".join(r["Kernel_Name"] for r in c)
        fp8 = "_fp8_kernel" in names or "grouped_gemm_kernel<true, true" in names
        # W_down packed to fp16: the down kernels' last template argument is true
        packed = bool(re.search(r"(grouped_gemm_kernel<false, false|down_stream_lds_kernel<[^>]*), true>", names))
        wl = ("prefill" if "grouped_gemm" in names else "decode") + ("_fp8" if fp8 else "") + \
            ("_packed" if packed else "")
        return wl + (", residual sublayer" if "prenorm_kernel" in names else "")

    per = {}
    for c in calls:
        wl = kind(c)
        for r in c:
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per.setdefault(wl, {}).setdefault(short(r["Kernel_Name"]), []).append(us)
    out = ["# rocprofv3 kernel times: Beam MoE block forward, decode T=64 and prefill T=16384, bf16 and FP8 weights",
           "", "Command (repository root on the GPU host):", "", "```",
           "cd /tmp && export TMPDIR=/tmp",
           "rocprofv3 --kernel-trace --stats --output-format csv -d <TRACE_DIR> -o run -- \\",
           f"    python3 $REPO/bench.py --workloads {TRACE_WORKLOADS} --steps 10 --warmup 2 --no-cpu-baseline",
           "python3 bench.py --summarize-trace <TRACE_DIR> <this file>", "```", "",
           "Calls are cut before each router_logits_kernel dispatch (before the prenorm_kernel of a",
           "residual-sublayer call); calls that ran the grouped GEMM are prefill, the others decode, with",
           "the suffix _fp8 where the FP8 kernels ran and _packed where the down kernel took W_down packed",
           "to fp16 (beam_moe_forward_packed).  Warmup and timed calls, with and without the stage",
           "markers, are all counted.  Durations are the dispatch end minus start timestamps.", ""]
    order = ["decode", "prefill", "prefill_packed", "decode_fp8", "prefill_fp8", "decode, residual sublayer",
             "prefill, residual sublayer"]
    for wl in order + sorted(k for k in per if k not in order):
        if wl not in per:
            continue
        ks = per[wl]
        total = sum(sum(v) for v in ks.values()) / max(len(v) for v in ks.values())
        out += [f"## {wl}", "", "| kernel | dispatches | average (us) | min (us) | max (us) | share |",
                "|---|---|---|---|---|---|"]
        for k, v in sorted(ks.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
            avg = sum(v) / len(v)
            out.append(f"| `{k}` | {len(v)} | {avg:.1f} | {min(v):.1f} | {max(v):.1f} | "
                       f"{100 * sum(v) / len(v) / total:.1f}% |")
        out.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def measured_traffic(workload):
    """Scaled HBM bytes per gate/up launch, if measured on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    sha = kernel_source_hash()
    for ln in text.splitlines():
        if ln.startswith("#") or not ln.strip():
            continue
        kv = dict(tok.split("=", 1) for tok in ln.split() if "=" in tok)
        if kv.get("workload") == workload and kv.get("source_sha") == sha:
            return int(kv["traffic_bytes"])
    return None


_PACKED = {}   # W_down packed to fp16 once per run (a weight-load step, outside every timed region)


def time_workload(name, experts, steps, warmup, experts_fp8=None):
    """`name` is a workload of synth.WORKLOADS, or one with the suffix "_fp8": the same batch
    through the FP8-weight entry point, or "_packed": the same batch through
    beam_moe_forward_packed, with W_down converted to fp16 once beforehand."""
    from grouped_top_routing_fp32_amd import binding, synth
    if name.endswith("_fp8"):
        return time_wl(synth.WORKLOADS[name[:-4]], experts, steps, warmup, fp8=experts_fp8)
    if name.endswith("_packed"):
        wl = synth.WORKLOADS[name[:-7]]
        if "wd" not in _PACKED:
            _PACKED["wd"] = binding.beam_moe_pack_weights(wl.dims, experts[2])
        return time_wl(wl, experts, steps, warmup, packed_down=_PACKED["wd"])
    return time_wl(synth.WORKLOADS[name], experts, steps, warmup)


def time_router_dispatch(steps, warmup):
    """Router + group-limited selection + dispatch alone on the router_dispatch workload
    (T = 4096 at Beam dims), through beam_moe_route and beam_moe_dispatch."""
    import torch
    from grouped_top_routing_fp32_amd import binding, synth

    wl = synth.WORKLOADS["router_dispatch"]
    d = wl.dims
    x = synth.make_x(wl, "cuda")
    wr = synth.make_router(wl, "cuda")
    ws = binding.workspace(d, wl.tokens, "cuda")
    st = torch.cuda.current_stream()

    def call():
        ids, _, _ = binding.beam_moe_route(d, x, wr, ws=ws, stream=st)
        binding.beam_moe_dispatch(d, ids, ws=ws, stream=st)

    for _ in range(warmup):
        call()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(st)
    for _ in range(steps):
        call()
    end.record(st)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    T, H, E = wl.tokens, d.hidden, d.num_experts
    flops = 2 * T * H * E
    return {"value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "config": {"workload": f"router_dispatch: router, selection and dispatch, T={T}", "tokens": T,
                       "hidden": H, "experts": E, "groups": d.num_groups, "topk_groups": d.topk_groups,
                       "topk": d.topk},
            "router_tflops_fp32_equivalent": round(flops / ms / 1e9, 2),
            "algorithmic_bytes": T * H * 2 + E * H * 4 + T * d.topk * 4 * 4}


def timed_loops(call, steps, warmup, stream):
    """Milliseconds of `steps` back-to-back calls (stage markers off), then the per-stage
    device times summed over a second loop of `steps` calls with the markers on (each
    marker costs a few microseconds of its own, so the first loop gives the step time)."""
    import torch
    from grouped_top_routing_fp32_amd import binding

    for _ in range(warmup):
        call()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    binding.beam_moe_timing_read()                 # drop anything recorded before
    binding.beam_moe_timing_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    binding.beam_moe_timing_enable(False)
    stage_ms, calls = binding.beam_moe_timing_read()
    assert calls == steps, (calls, steps)
    return total_ms, stage_ms


def time_wl(wl, experts, steps, warmup, fp8=None, packed_down=None):
    import torch
    from grouped_top_routing_fp32_amd import binding, synth

    d = wl.dims
    x = synth.make_x(wl, "cuda")
    wr = synth.make_router(wl, "cuda")
    bias = synth.make_bias(wl, "cuda")
    wg, wu, wd = experts if fp8 is None else (None, None, None)
    bufs = binding.ForwardBuffers(d, wl.tokens, "cuda")
    stream = torch.cuda.current_stream()
    if fp8 is not None:
        call = lambda: binding.beam_moe_forward_fp8(d, x, wr, bias, *fp8, bufs=bufs, stream=stream)  # noqa: E731
    elif packed_down is not None:
        call = lambda: binding.beam_moe_forward_packed(d, x, wr, bias, wg, wu, packed_down,  # noqa: E731
                                                       bufs=bufs, stream=stream)
    else:
        call = lambda: binding.beam_moe_forward(d, x, wr, bias, wg, wu, wd, bufs=bufs, stream=stream)  # noqa: E731
    total_ms, stage_ms = timed_loops(call, steps, warmup, stream)
    counts = bufs.counts.cpu()
    return dict(wl=wl, total_ms=total_ms, ms_per_step=total_ms / steps,
                stage_ms={k: v / steps for k, v in stage_ms.items()},
                n_touched=int((counts > 0).sum()), max_count=int(counts.max()), x=x, wr=wr, bias=bias, bufs=bufs)


def time_residual(r, steps, warmup):
    """The same batch through the residual-sublayer entry point (pre-norm, block, post-norm, scaled
    update at step 2, unit norm weights), out of place so every step sees the same stream."""
    import torch
    from grouped_top_routing_fp32_amd import binding, synth

    wl = r["wl"]
    d = wl.dims
    stream_in = synth.make_stream(wl, "cuda")
    wg, wu, wd = r["experts"]
    bufs = binding.ForwardBuffers(d, wl.tokens, "cuda")
    st = torch.cuda.current_stream()
    call = lambda: binding.beam_moe_residual_forward(d, stream_in, 2, r["wr"], r["bias"], wg, wu, wd,  # noqa: E731
                                                     bufs=bufs, stream=st)
    total_ms, stage_ms = timed_loops(call, steps, warmup, st)
    ms = total_ms / steps
    stage = {k: round(v / steps, 4) for k, v in stage_ms.items()}
    touched = int((bufs.counts > 0).sum())
    T, H = wl.tokens, d.hidden
    # over the plain block: the pre-norm reads the fp32 stream and writes bf16 x (6 bytes per
    # element), the fused combine also reads the stream (4)
    extra_bytes = T * H * 10
    # the cost of the sublayer's own work, free of the routing difference (the normalised stream
    # routes to a different set of experts than the block's own x): pre-norm plus the fused
    # combine's time above the plain combine's
    own_ms = stage["prenorm"] + stage["combine"] - r["stage_ms"]["combine"]
    return {"ms_per_step": round(ms, 4), "value": round(T / (ms / 1e3), 1), "unit": "tokens/s",
            "stage_ms": stage, "experts_touched": touched,
            "norm_and_update_ms": round(own_ms, 4),
            "extra_algorithmic_bytes": extra_bytes, "step": 2, "norm": "RMSNorm, eps 1e-6, unit weights"}


# The arithmetic types of the path (include/beam_moe.h states the same).
DTYPE_BF16 = "mixed bf16/fp16/fp32"
DTYPE_FP8 = "mixed e4m3 weights, bf16/fp16/fp32"
PRECISION = {
    "weights": "bf16 (fp8 records: E4M3 codes with an fp32 scale per output row)",
    "router": "fp32 (bf16 x times fp32 W_r, FP32 accumulation); selection and weights fp32",
    "gate_up": "bf16 MFMA, fp32 accumulation, SwiGLU in fp32",
    "h": "fp16 times 2^-s per 64 columns of a row group",
    "down": "fp16 MFMA on W_down converted exactly to fp16, fp32 accumulation",
    "y": "fp16 times 2^-s per 64 columns of a row group",
    "combine_out": "fp32",
}


def accounting(r):
    """Algorithmic bytes and FLOPs of each kernel of one step (no cache effects, no re-reads)."""
    wl = r["wl"]
    d = wl.dims
    T, H, I, E, K = wl.tokens, d.hidden, d.intermediate, d.num_experts, d.topk
    n = T * K
    nt = r["n_touched"]
    # weight bytes per element: bf16, or E4M3 codes plus an fp32 scale per row
    wb = 1 if r.get("fp8") else 2
    srow = 4 if r.get("fp8") else 0
    b = {
        "router_logits": T * H * 2 + E * H * 4,
        "gate_up": nt * 2 * I * (H * wb + srow) + T * H * 2 + n * I * 2,
        "down": nt * H * (I * wb + srow) + n * I * 2 + n * H * 2 + n * (H // 64),
        "combine": n * H * 2 + n * (H // 64) + n * 4 + T * H * 4,
    }
    f = {
        "router_logits": 2 * T * H * E,
        "gate_up": 2 * n * 2 * I * H,
        "down": 2 * n * H * I,
    }
    layer_bytes = nt * 3 * I * H * wb + nt * (2 * I + H) * srow + E * H * 4 + T * H * 2 + T * H * 4
    expert_flops = 2 * n * 3 * I * H
    return b, f, layer_bytes, expert_flops


def roofline(r, bound, name):
    b, f, layer_bytes, expert_flops = accounting(r)
    kernel = "gate_up"
    dur_s = r["stage_ms"][kernel] / 1e3
    traffic = measured_traffic(name)
    if bound == "hbm":
        achieved = b[kernel] / dur_s / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": b[kernel], "avg_launch_ms": round(r["stage_ms"][kernel], 4)}
    achieved = f[kernel] / dur_s / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "algorithmic_flops_per_launch": f[kernel], "algorithmic_bytes_per_launch": b[kernel],
            "avg_launch_ms": round(r["stage_ms"][kernel], 4)}


def layer_summary(r):
    b, f, layer_bytes, expert_flops = accounting(r)
    s = r["ms_per_step"] / 1e3
    return {"layer_hbm_gbs": round(layer_bytes / s / 1e9, 1), "layer_hbm_frac": round(layer_bytes / s / 1e9 / HBM_PEAK_GBS, 4),
            "layer_expert_tflops": round(expert_flops / s / 1e12, 1),
            "layer_mfma_frac": round(expert_flops / s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
            "experts_touched": r["n_touched"], "max_rows_per_expert": r["max_count"]}


_HOST_EXPERTS = {}   # host copies of expert weights, shared by the baselines of one run


def cpu_baseline(r, target_s, seed=0):
    """The FP64 oracle on the host cores, on a seeded random subset of the same batch.

    The oracle runs the whole block (router, selection, dispatch, experts, combine) on
    n tokens, n sized from an untimed one-token pilot so that the run takes about
    target_s.  Expert weights are copied to the host before the timed region; inside
    it the oracle reads them as it always does (bf16 values widened to FP64, or E4M3
    codes decoded and scaled by their row scales)."""
    import numpy as np
    import torch
    from oracle import beam_moe_oracle as orc
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info if i.get("user_api") == "blas"}))
    except Exception:
        blas_threads, blas = os.cpu_count(), "?"
    wl = r["wl"]
    d = wl.dims
    fp8 = r.get("fp8")
    X_all = r["x"].float().cpu().numpy()
    W_r = r["wr"].cpu().numpy()
    bias = None if r["bias"] is None else r["bias"].cpu().numpy()
    src = r["experts_fp8"] if fp8 else r["experts"]
    e4m3 = orc.e4m3_decode(np.arange(256)) if fp8 else None

    def fetch(ids):
        for e in np.unique(ids):
            key = (bool(fp8), int(e))
            if key not in _HOST_EXPERTS:
                _HOST_EXPERTS[key] = tuple(t[int(e)].cpu() for t in src)

    def weights(e):
        h = _HOST_EXPERTS[(bool(fp8), int(e))]
        if fp8:
            # W = decode(q) * row scale: the oracle's value of each of the 256 codes, looked up
            return tuple(e4m3[q.numpy()] * sc.numpy().astype(np.float64)[:, None]
                         for q, sc in ((h[0], h[1]), (h[2], h[3]), (h[4], h[5])))
        return tuple(t.float().numpy() for t in h)

    def run(tok):
        ids, *_ = orc.route(X_all[tok], W_r, bias, d.num_groups, d.topk_groups, d.topk, d.routed_scaling)
        fetch(ids)
        t0 = time.perf_counter()
        orc.moe_forward(X_all[tok], W_r, bias, weights, d.num_groups, d.topk_groups, d.topk, d.routed_scaling)
        return time.perf_counter() - t0

    rng = np.random.default_rng(seed)
    per_token = run(rng.choice(wl.tokens, 1, replace=False))     # untimed pilot
    n = int(max(1, min(wl.tokens, target_s / max(per_token, 1e-3))))
    tok = np.sort(rng.choice(wl.tokens, n, replace=False))
    el = run(tok)
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{n} of the {wl.tokens} tokens of the {wl.name} batch (seeded random subset, seed {seed})"
                      f"{' with FP8 expert weights' if fp8 else ''}, whole block in FP64 "
                      f"(numpy, BLAS={blas}); {el:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def expert_path(wl, fp8=False):
    """Which expert kernels the library runs for this batch, as it reports them."""
    from grouped_top_routing_fp32_amd import binding
    rows = binding.beam_moe_stream_rows(wl.dims, wl.tokens, fp8)
    return f"stream, {rows}-row tiles" if rows else "grouped GEMM"


def sweep(args, experts, experts_fp8=None):
    """Tokens/s and both roofline fractions of the whole layer over batch sizes T (bf16 experts,
    or FP8 ones through the FP8-weight entry point)."""
    from grouped_top_routing_fp32_amd import synth
    base = synth.WORKLOADS["decode"]
    points = []
    for T in [int(t) for t in args.sweep_tokens.split(",") if t]:
        wl = synth.with_tokens(base, T)
        steps = max(3, min(args.steps, int(2000 / max(1, T))))  # keep large batches short
        r = time_wl(wl, experts, steps, args.warmup, fp8=experts_fp8)
        r["fp8"] = experts_fp8 is not None
        s = layer_summary(r)
        hbm, mfma = s["layer_hbm_frac"], s["layer_mfma_frac"]
        points.append({"T": T, "steps": steps, "ms_per_step": round(r["ms_per_step"], 4),
                       "tokens_per_s": round(T / (r["ms_per_step"] / 1e3), 1),
                       "path": expert_path(wl, experts_fp8 is not None),
                       "experts_touched": r["n_touched"], "max_rows_per_expert": r["max_count"],
                       "layer_hbm_gbs": s["layer_hbm_gbs"], "layer_hbm_frac": hbm,
                       "layer_expert_tflops": s["layer_expert_tflops"], "layer_mfma_frac": mfma,
                       "bound": "hbm" if hbm >= mfma else "mfma", "stage_ms": s["stage_ms"]})
        print(f"[bench] sweep T={T}: {r['ms_per_step']:.4f} ms, hbm {hbm:.3f}, mfma {mfma:.3f}",
              file=sys.stderr, flush=True)
    print(json.dumps({"metric": "MoE-layer tokens/s and roofline fractions over batch size T", "unit": "tokens/s",
                      "n_gpus": 1, "dtype": DTYPE_FP8 if experts_fp8 is not None else DTYPE_BF16,
                      "data": "synthetic",
                      "config": {"workload": "Beam MoE block forward, T swept", "hidden": base.dims.hidden,
                                 "intermediate": base.dims.intermediate, "experts": base.dims.num_experts,
                                 "topk": base.dims.topk,
                                 "weights": "e4m3 + fp32 row scales" if experts_fp8 is not None else "bf16"},
                      "points": points}), flush=True)


COUNTER_SET = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
               "SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_LDS_DATA_FIFO_FULL GRBM_GUI_ACTIVE")


def summarize_counters(out_md, *passes):
    """Per-kernel means of every counter of rocprofv3 --pmc runs of this script, plus the derived
    MFMA-busy and wave-wait fractions where their counters were collected.  Each pass is
    WORKLOADS=COUNTER_DIR: one run with --workloads WORKLOADS, so that workloads whose kernels share
    a name (prefill and skewed) are summarised apart."""
    import csv
    import glob
    simds, xcds = 256 * 4, 8
    sections, cmds = [], []
    for spec in passes:
        workloads, counter_dir = spec.split("=", 1)
        cmds.append(f"rocprofv3 --pmc {COUNTER_SET} --kernel-include-regex 'beam::' --output-format csv "
                    f"-d <COUNTER_DIR_{len(cmds) + 1}> -o run "
                    f"-- python3 bench.py --workloads {workloads} --steps 2 --warmup 1 --no-cpu-baseline --no-residual")
        per, order = {}, []
        for path in sorted(glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True)):
            with open(path) as f:
                disp = {}
                for r in csv.DictReader(f):
                    if "beam::" not in r["Kernel_Name"]:
                        continue
                    d = disp.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"]})
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                for d in disp.values():
                    name = d.pop("kernel").replace("void ", "")
                    name = name[:name.index("(")] if "(" in name else name
                    if name not in per:
                        order.append(name)
                    per.setdefault(name, []).append(d)
        for name in order:
            rows = per[name]
            keys = sorted({k for d in rows for k in d})
            mean = {k: sum(d.get(k, 0.0) for d in rows) / len(rows) for k in keys}
            sec = [f"## {workloads}: `{name}` ({len(rows)} dispatches)", "", "| counter | mean per dispatch |",
                   "|---|---|"]
            sec += [f"| {k} | {mean[k]:.4g} |" for k in keys]
            if mean.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (mean["GRBM_GUI_ACTIVE"] / xcds)
                sec.append(f"| MFMA busy (derived) | {busy:.3f} |")
            if mean.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in mean:
                sec.append(f"| wave wait (derived) | {mean['SQ_WAIT_ANY'] / mean['SQ_WAVE_CYCLES']:.3f} |")
            sections += sec + [""]
    out = ["# rocprofv3 counters per kernel: Beam MoE block forward, decode T=64, prefill T=16384, "
           "skewed T=8192", "",
           "Commands (repository root on the GPU host, after `cd /tmp && export TMPDIR=/tmp`), one counter run per "
           "line of workloads:", "", "```"] + cmds + [
           "python3 bench.py --summarize-counters <this file> " +
           " ".join(f"{spec.split('=', 1)[0]}=<COUNTER_DIR_{i + 1}>" for i, spec in enumerate(passes)), "```", "",
           "Values are per dispatch, each counter summed over the dimensions rocprofv3 reports it in, then",
           "averaged over the dispatches.  Derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x",
           "GRBM_GUI_ACTIVE / 8 XCDs), the share of every SIMD's cycles its matrix unit was busy; wave wait =",
           "SQ_WAIT_ANY / SQ_WAVE_CYCLES, the share of wave time spent waiting (on memory counters or a barrier).",
           ""] + sections
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def gemm_reference():
    """Context for the prefill GEMMs: the platform's GEMM library (torch.bmm / linear on bf16,
    contiguous operands) on the MoE shapes of the prefill batch, 256 experts x 512 rows."""
    import torch
    E, R, H, I = 256, 512, 5120, 2560

    def t(fn, flops, name):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 10
        return {"case": name, "ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 1),
                "frac_of_bf16_peak": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}

    g = torch.Generator(device="cuda").manual_seed(0)
    res = []
    a = torch.randn(E, R, H, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(E, H, 2 * I, device="cuda", dtype=torch.bfloat16, generator=g)
    res.append(t(lambda: torch.bmm(a, b), 2 * E * R * H * 2 * I, "bmm 256 x (512x5120 @ 5120x5120): gate/up shape"))
    del a, b
    a = torch.randn(E, R, I, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(E, I, H, device="cuda", dtype=torch.bfloat16, generator=g)
    res.append(t(lambda: torch.bmm(a, b), 2 * E * R * I * H, "bmm 256 x (512x2560 @ 2560x5120): down shape"))
    del a, b
    a = torch.randn(E * R, H, device="cuda", dtype=torch.bfloat16, generator=g)
    w = torch.randn(2 * I, H, device="cuda", dtype=torch.bfloat16, generator=g)
    res.append(t(lambda: torch.nn.functional.linear(a, w), 2 * E * R * H * 2 * I,
                 "linear 131072x5120 @ (5120x5120)^T: one dense GEMM of the same work"))
    del a, w
    torch.cuda.empty_cache()
    print(json.dumps({"gemm_reference": res}), flush=True)


def copy_calibration():
    """A plain elementwise copy of COPY_BYTES (read once, written once), outside any timed region."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_sweep:
        summarize_sweep(*args.summarize_sweep)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Beam MoE block here runs on a single MI355X "
              "(no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from grouped_top_routing_fp32_amd import binding, synth
    binding.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.gemm_reference:
        gemm_reference()
        return
    names = [w for w in args.workloads.split(",") if w]
    print(f"[bench] generating Beam expert weights (20.1 GB bf16) on the device", file=sys.stderr, flush=True)
    experts = None if (args.sweep and args.sweep_fp8) else synth.make_experts(synth.WORKLOADS["decode"], "cuda")
    experts_fp8 = None
    if (any(n.endswith("_fp8") for n in names) and not args.sweep) or (args.sweep and args.sweep_fp8):
        print(f"[bench] generating Beam FP8 expert weights (10.1 GB E4M3 + row scales) on the device",
              file=sys.stderr, flush=True)
        experts_fp8 = synth.make_experts_fp8(synth.WORKLOADS["decode"], "cuda")
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()
    if args.sweep:
        sweep(args, experts, experts_fp8 if args.sweep_fp8 else None)
        return
    results = {}
    extra = {}
    if "router_dispatch" in names:
        names = [n for n in names if n != "router_dispatch"]
        print("[bench] timing router_dispatch", file=sys.stderr, flush=True)
        extra["router_dispatch"] = time_router_dispatch(args.steps, args.warmup)
    for name in names:
        print(f"[bench] timing {name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
        r = time_workload(name, experts, args.steps, args.warmup, experts_fp8)
        r["experts"] = experts
        r["experts_fp8"] = experts_fp8
        r["fp8"] = name.endswith("_fp8")
        r["packed"] = name.endswith("_packed")
        results[name] = r
        print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step; stages {r['stage_ms']}", file=sys.stderr, flush=True)
        if not args.no_residual and not r["fp8"] and not r["packed"]:
            r["residual"] = time_residual(r, args.steps, args.warmup)
            print(f"[bench] {name} as a residual sublayer: {r['residual']['ms_per_step']:.4f} ms/step",
                  file=sys.stderr, flush=True)

    head = names[0]

    def record(name):
        r = results[name]
        wl = r["wl"]
        d = wl.dims
        bound = "hbm" if wl.tokens * d.topk / d.num_experts < 32 else "mfma"
        what = "Beam MoE block forward" + (" with FP8 E4M3 expert weights" if r["fp8"] else "") + \
            (" with W_down packed to fp16 once (beam_moe_pack_weights; bf16 gate/up)" if r["packed"] else "")
        cfg = {"workload": f"{name}: {what}, T={wl.tokens}", "tokens": wl.tokens,
               "hidden": d.hidden, "intermediate": d.intermediate, "experts": d.num_experts,
               "groups": d.num_groups, "topk_groups": d.topk_groups, "topk": d.topk,
               "routed_scaling": d.routed_scaling, "router_bias": "zipf(1.2)" if wl.zipf_s else None}
        out = {"value": round(wl.tokens / (r["ms_per_step"] / 1e3), 1), "unit": "tokens/s",
               "ms_per_step": round(r["ms_per_step"], 4), "config": cfg, "roofline": roofline(r, bound, name)}
        out.update(layer_summary(r))
        out["dtype"] = DTYPE_FP8 if r["fp8"] else DTYPE_BF16
        if "residual" in r:
            out["residual_sublayer"] = r["residual"]
        if not args.no_cpu_baseline and name != head and not r["packed"]:
            print(f"[bench] cpu baseline (oracle) on {name}", file=sys.stderr, flush=True)
            out["cpu_baseline"] = cpu_baseline(r, args.cpu_seconds / 2)
        return out

    line = {"metric": METRIC}
    main_rec = record(head)
    line.update({"value": main_rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                 "warmup": args.warmup, "ms_per_step": main_rec["ms_per_step"], "higher_is_better": True,
                 "scaling": "weak", "vs_baseline": None, "dtype": main_rec["dtype"], "precision": PRECISION,
                 "data": "synthetic",
                 "config": main_rec["config"], "roofline": main_rec["roofline"]})
    for k in ("layer_hbm_gbs", "layer_hbm_frac", "layer_expert_tflops", "layer_mfma_frac", "stage_ms",
              "experts_touched", "max_rows_per_expert", "residual_sublayer"):
        if k not in main_rec:
            continue
        line[k] = main_rec[k]
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle) on {head}", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(results[head], args.cpu_seconds)
    for name in names[1:]:
        line[name] = record(name)
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
