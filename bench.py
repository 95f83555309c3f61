"""Benchmark of the weight-only-quantized MoE layer on one MI355X.

One step = one layer call on one batch, from router logits to the output:
softmax top-k routing, align, GEMM1 + SiLU-and-mul, GEMM2 and the weighted
combine (moe_w8a16_apply / moe_w4a16_apply), inputs resident in HBM.  Weight
quantization runs once at set-up and is not part of a step.

Default workload: the Mixtral-shaped decode batch (E=8, top-2, H=4096,
I=14336, int8 per-channel weights, bf16 activations) at T=64 tokens.
--weights fp8 (e4m3fn weights, moe_wfp8a16_apply) and --weights w8a8 (int8
weights and per-token int8 activations, moe_w8a8_apply) measure the other
expert formats on the same workloads.

Prints one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (from HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "weight_quantized_mixture_amd", "csrc")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_decode",
                    choices=["tiny", "mixtral_decode", "mixtral_prefill", "fine_grained", "w4a16"])
    ap.add_argument("--tokens", type=int, default=None, help="T (default: the workload's headline size)")
    ap.add_argument("--weights", default="int8", choices=["int8", "fp8", "w8a8"],
                    help="expert format of the int8 workloads: int8 per-channel weights with 16-bit activations "
                         "(the default), fp8 e4m3fn weights with one scale per expert and matrix, or int8 "
                         "weights with int8 activations quantized per token (W8A8)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (3 times) and exit: the known "
                         "byte count that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of a bench run, then of "
                         "--calibrate-copy-mb 1024) into the traffic summary under profiles/ and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the traffic summary")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc output folder with SQ/GRBM counters into the per-kernel busy "
                         "summary under profiles/ and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats output folder into the kernel-time summary "
                         "under profiles/ and exit")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="read this many MB of other data between timed steps (outside the events) so "
                         "the 256 MB Infinity Cache does not serve the weights (0 = no flush).  A read, "
                         "not a write: written lines would be written back to HBM during the next timed step")
    ap.add_argument("--no-prefill-band", action="store_true",
                    help="with the default decode workload, skip the Mixtral prefill T=4096 line measured "
                         "next to it on the same weights")
    return ap.parse_args()


# the metric's MFMA band, measured next to the default decode line
PREFILL_BAND_T = 4096

HEADLINE_T = {"tiny": 16, "mixtral_decode": 64, "mixtral_prefill": 4096, "fine_grained": 512, "w4a16": 256}


# source file of each GEMM1 kernel whose traffic the bench reports
KERNEL_SOURCE = {"gemm1_big_kernel": "gemm_w8_big.hip", "gemm1_dma_kernel": "gemm_w8_dma.hip",
                 "gemm1_lds_kernel": "gemm_w8_lds.hip", "gemm1_stream_kernel": "gemm_w8_stream.hip",
                 "gemm1_w8_kernel": "gemm_w8.hip"}


def sources_sha(kernel_prefix=None) -> str:
    """Hash of the HIP sources a kernel is built from (its .hip file and the headers with device
    code; launch.hpp only declares host launchers; every source without a kernel): a traffic
    summary is valid only for the kernels it was taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    hips = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if kernel_prefix in KERNEL_SOURCE:
        hips = [os.path.join(CSRC, KERNEL_SOURCE[kernel_prefix])]
    headers = [f for f in sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) if os.path.basename(f) != "launch.hpp"]
    for f in hips + headers:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _pmc_rows(folder):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    out = {}
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"]
        out.setdefault((name, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(args):
    """Traffic of every library kernel per launch, scaled by what the counters read for a copy of known size."""
    fetch, write = _pmc_rows(args.summarize_pmc[0]), _pmc_rows(args.summarize_pmc[1])
    cf, cw = _pmc_rows(args.summarize_pmc[2]), _pmc_rows(args.summarize_pmc[3])
    copy_bytes = 1024 << 20

    def copy_kib(rows, counter):
        v = [x for (n, c), xs in rows.items() if c == counter and "copyBuffer" in n for x in xs]
        if not v:
            v = [x for (n, c), xs in rows.items() if c == counter and "copy" in n.lower() for x in xs]
        return max(v)
    f_scale = (copy_bytes / 1024) / copy_kib(cf, "FETCH_SIZE")
    w_scale = (copy_bytes / 1024) / copy_kib(cw, "WRITE_SIZE")
    kernels = {}
    for (name, c), xs in fetch.items():
        if c == "FETCH_SIZE" and "moe::" in name:
            kernels.setdefault(name, {})["fetch_kib"] = sum(xs) / len(xs)
    for (name, c), xs in write.items():
        if c == "WRITE_SIZE" and "moe::" in name:
            kernels.setdefault(name, {})["write_kib"] = sum(xs) / len(xs)
    res = {"sources_sha": sources_sha(), "kernel_sources_sha": {k: sources_sha(k) for k in KERNEL_SOURCE},
           "fetch_scale": f_scale, "write_scale": w_scale,
           "command": args.pmc_command, "workload": args.workload,
           "T": args.tokens or HEADLINE_T[args.workload], "kernels": {}}
    lines = [f"# HBM traffic per launch: {args.workload}, T={res['T']}", "",
             f"Command: `{args.pmc_command}`", "",
             f"Copy calibration: a 1 GiB copy reads {copy_bytes / 1024 / f_scale:.0f} KiB in FETCH_SIZE "
             f"(scale x{f_scale:.3f}) and writes {copy_bytes / 1024 / w_scale:.0f} KiB in WRITE_SIZE (scale x{w_scale:.3f}).",
             "", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled traffic MB |", "|---|---|---|---|"]
    for name, d in sorted(kernels.items()):
        fk, wk = d.get("fetch_kib", 0.0), d.get("write_kib", 0.0)
        mb = (fk * f_scale + wk * w_scale) * 1024 / 1e6
        short = name.replace("moe::(anonymous namespace)::", "").replace("void ", "").split("(moe::")[0][:90]
        res["kernels"][short] = {"fetch_kib": fk, "write_kib": wk, "traffic_bytes": mb * 1e6}
        lines.append(f"| `{short}` | {fk:.0f} | {wk:.0f} | {mb:.1f} |")
    lines += ["", f"Kernel sources sha256[:16]: `{res['sources_sha']}` (all); per GEMM1 kernel: " +
              ", ".join(f"`{k}` `{v}`" for k, v in res["kernel_sources_sha"].items())]
    stem = f"traffic_{args.workload}_T{res['T']}{fmt_suffix(args)}"
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(res, open(os.path.join(PROFILES, stem + ".json"), "w"), indent=1)
    open(os.path.join(PROFILES, stem + ".md"), "w").write("\n".join(lines) + "\n")
    print(json.dumps(res), flush=True)


def fmt_suffix(args) -> str:
    """File-name suffix of a summary: the expert format unless it is the default int8."""
    return "" if args.weights == "int8" else f"_{args.weights}"


def summarize_trace(args):
    import csv
    import glob
    files = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.summarize_trace}")
    T = args.tokens or HEADLINE_T[args.workload]
    lines = [f"# Kernel times: {args.workload}, T={T}, {args.weights} experts", "", f"Command: `{args.pmc_command}`", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(files[0])):
        name = r["Name"].replace("moe::(anonymous namespace)::", "").replace("void ", "")
        name = name.split("(moe::")[0].split("(float const")[0].split("(int const")[0][:90]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"Kernel sources sha256[:16]: `{sources_sha()}`"]
    stem = f"kernels_{args.workload}_T{T}{fmt_suffix(args)}"
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, stem + ".md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def summarize_counters(args):
    """Per-kernel busy fractions from SQ counters (summed over the SIMDs / XCDs of the chip)."""
    rows = _pmc_rows(args.summarize_counters)
    T = args.tokens or HEADLINE_T[args.workload]
    kernels = {}
    for (name, c), xs in rows.items():
        if "moe::" not in name:
            continue
        short = name.replace("moe::(anonymous namespace)::", "").replace("void ", "").split("(moe::")[0]
        short = short.split("(float const")[0].split("(int const")[0][:70]
        kernels.setdefault(short, {})[c] = sum(xs) / len(xs)
    lines = [f"# SQ counters per launch: {args.workload}, T={T}", "", f"Command: `{args.pmc_command}`", "",
             "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the kernel's GPU cycles are GRBM_GUI_ACTIVE / 8; "
             "SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs.", "",
             "| kernel | GPU cycles | MFMA busy (per SIMD) | VALU active / wave cycles | waiting / wave cycles | "
             "LDS bank conflicts |", "|---|---|---|---|---|---|"]
    for name, m in sorted(kernels.items()):
        cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        wave = m.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024.0 / cyc if cyc else 0.0
        lines.append(f"| `{name}` | {cyc:.0f} | {100 * busy:.1f}% | "
                     f"{100 * m.get('SQ_ACTIVE_INST_VALU', 0.0) / wave:.1f}% | "
                     f"{100 * m.get('SQ_WAIT_INST_ANY', 0.0) / wave:.1f}% | {m.get('SQ_LDS_BANK_CONFLICT', 0.0):.3g} |")
    lines += ["", f"Kernel sources sha256[:16]: `{sources_sha()}`"]
    stem = f"counters_{args.workload}_T{T}{fmt_suffix(args)}"
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, stem + ".md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def recorded_traffic(workload, T, kernel_prefix):
    """Scaled HBM bytes of the dominant kernel from the committed summary, if the kernels are unchanged."""
    path = os.path.join(PROFILES, f"traffic_{workload}_T{T}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_sources_sha", {}).get(kernel_prefix) != sources_sha(kernel_prefix):
        return None
    for name, v in d["kernels"].items():
        if name.startswith(kernel_prefix):
            return v["traffic_bytes"]
    return None


def _rnd(v, n=5):
    """Round floats for the JSON line (keeps it short enough for a log tail)."""
    if isinstance(v, float):
        return float(f"{v:.{n}g}")
    if isinstance(v, dict):
        return {k: _rnd(x, n) for k, x in v.items()}
    return v


def measure(pkg, synthetic, torch, dev, layer, wl, T, args, want_stages=True, fmt="int8"):
    """Time `args.steps` layer calls (logits -> output) of workload `wl` at T tokens on the layer's
    resident weights, with a read flush of `args.flush_mb` MB before each step (outside the timed
    events), then (int8 weights with 16-bit activations) time each stage once per repetition for the
    dominant kernel's roofline; the other formats report the whole layer against the roofline of
    their arithmetic."""
    import numpy as np
    E, k, H, I = wl.E, wl.k, wl.H, wl.I
    w4 = wl.weights == "w4"
    xb = synthetic.activations(wl, T, args.seed)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16 if wl.act == "bf16" else torch.float16).to(dev)
    logits_np = synthetic.router_logits(wl, T, args.seed)
    logits = torch.from_numpy(logits_np).to(dev)
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    ti = torch.empty(T, k, dtype=torch.int32, device=dev)
    block_m = pkg.moe_w8a16_block_m(T, H, I, E, k)
    splits = pkg.moe_w8a16_splits(T, H, I, E, k, block_m)
    ws_fn = {"int8": pkg.moe_w8a16_workspace_bytes, "fp8": pkg.moe_wfp8a16_workspace_bytes,
             "w8a8": pkg.moe_w8a8_workspace_bytes}[fmt]
    ws_bytes = (pkg.moe_w4a16_workspace_bytes if w4 else ws_fn)(T, H, I, E, k, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        # logits -> output in one library call (routing, align, GEMM1+SiLU, GEMM2, combine)
        if w4:
            pkg.moe_w4a16_apply(x, logits, wl.renormalize, layer.w13_qweight, layer.w13_scales, layer.w13_qzeros,
                                layer.w2_qweight, layer.w2_scales, layer.w2_qzeros, wl.group_size, tw, ti, out, ws,
                                0, stream)
        elif fmt == "fp8":
            pkg.moe_wfp8a16_apply(x, logits, layer.w13_weight, layer.w13_weight_scale, layer.w2_weight,
                                  layer.w2_weight_scale, tw, ti, out, ws, renormalize=wl.renormalize, stream=stream)
        elif fmt == "w8a8":
            pkg.moe_w8a8_apply(x, logits, layer.w13_weight, layer.w13_scale, layer.w2_weight, layer.w2_scale, tw,
                               ti, out, ws, renormalize=wl.renormalize, stream=stream)
        else:
            pkg.moe_w8a16_apply(x, logits, wl.renormalize, layer.w13_weight, layer.w13_scale, layer.w2_weight,
                                layer.w2_scale, tw, ti, out, ws, 0, stream)

    step()
    torch.cuda.synchronize()
    ids_np = ti.cpu().numpy()
    active = np.unique(ids_np[(ids_np >= 0) & (ids_np < E)])
    n_active = int(active.size)

    # algorithmic work (what the method must move / compute; padding, the a/y
    # round trips and the second (lo) MFMA of the intermediate are not counted)
    if w4:
        g = wl.group_size
        per_expert_w13 = (2 * I * H) // 2 + (2 * I * (H // g)) * 2 + (2 * I * (H // g)) // 2
        per_expert_w2 = (H * I) // 2 + (H * (I // g)) * 2 + (H * (I // g)) // 2
    elif fmt == "fp8":
        per_expert_w13 = 2 * I * H + 4
        per_expert_w2 = H * I + 4
    else:
        per_expert_w13 = 2 * I * H + 2 * I * 4
        per_expert_w2 = H * I + H * 4
    act_bytes = 2
    bytes_layer = (n_active * (per_expert_w13 + per_expert_w2) + T * H * act_bytes * 2 + T * E * 4 + T * k * 8)
    bytes_gemm1 = n_active * per_expert_w13 + T * H * act_bytes
    flops_layer = 6 * T * k * H * I
    flops_gemm1 = 4 * T * k * H * I

    flush_mb = args.flush_mb
    flush = torch.ones(flush_mb << 18, dtype=torch.int32, device=dev) if flush_mb else None
    flush_sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def evict():
        if flush is not None:
            torch.amax(flush, dim=0, keepdim=True, out=flush_sink)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = float(np.mean(step_ms))

    # per-kernel durations: the same kernels, one stage call at a time, HIP events on the launch stream
    stage_ms = {}
    if not w4 and want_stages and fmt == "int8":
        cap = pkg.moe_align_capacity(T, k, E, block_m)
        s_ids = torch.empty(cap, dtype=torch.int32, device=dev)
        b_exp = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
        npad = torch.empty(1, dtype=torch.int32, device=dev)
        a_buf = torch.empty(pkg.moe_w8a16_intermediate_bytes(T, H, I, E, k, block_m) // 4 + 64, dtype=torch.float32,
                            device=dev)
        y_buf = torch.empty(splits, T * k, H, dtype=torch.float32, device=dev)
        names = ["route", "align", "gemm1", "requant", "gemm2", "combine"]
        acc = {n: [] for n in names}
        reps = max(5, min(args.steps, 20))
        for i in range(reps + 2):
            evict()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
            ev[0].record(stream)
            pkg.moe_route_topk(logits, k, wl.renormalize, tw, ti, stream)
            ev[1].record(stream)
            pkg.moe_align_block(ti, E, block_m, s_ids, b_exp, npad, stream)
            ev[2].record(stream)
            pkg.moe_w8a16_gemm1(x, layer.w13_weight, layer.w13_scale, s_ids, b_exp, npad, block_m, k, a_buf, stream)
            ev[3].record(stream)
            pkg.moe_w8a16_requant(a_buf, T, I, E, k, s_ids, npad, block_m, stream)
            ev[4].record(stream)
            pkg.moe_w8a16_gemm2(a_buf, T, k, layer.w2_weight, layer.w2_scale, s_ids, b_exp, npad, block_m, splits,
                                y_buf, stream)
            ev[5].record(stream)
            pkg.moe_combine_topk(y_buf, splits, tw, ti, E, out, stream)
            ev[6].record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                for j, n in enumerate(names):
                    acc[n].append(ev[j].elapsed_time(ev[j + 1]))
        stage_ms = {n: float(np.mean(v)) for n, v in acc.items()}
        del a_buf, y_buf

    mfma_band = T >= 1024
    # W8A8 multiplies int8 by int8 on the MFMA (int8 peak); the other formats decode the weights
    # exactly into 16-bit MFMA operands (bf16/fp16 peak)
    mfma_peak, mfma_unit = (INT8_PEAK_TOPS, "TOP/s") if fmt == "w8a8" else (BF16_PEAK_TFLOPS, "TFLOP/s")
    layer_hbm_frac = bytes_layer / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS
    layer_mfma_frac = flops_layer / (ms_per_step / 1e3) / 1e12 / mfma_peak
    if stage_ms:
        dur_s = stage_ms["gemm1"] / 1e3
        if mfma_band:
            roof = {"bound": "mfma", "achieved": flops_gemm1 / dur_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": bytes_gemm1 / dur_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["kernel"] = gemm1_kernel_name(block_m, H)
        roof["traffic"] = recorded_traffic(wl.name, T, roof["kernel"])
        roof["kernel_ms"] = stage_ms["gemm1"]
    else:
        dur_s = ms_per_step / 1e3
        if mfma_band:
            roof = {"bound": "mfma", "achieved": flops_layer / dur_s / 1e12, "peak": mfma_peak, "unit": mfma_unit,
                    "frac": layer_mfma_frac, "traffic": None, "kernel": "whole layer"}
        else:
            roof = {"bound": "hbm", "achieved": bytes_layer / dur_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": layer_hbm_frac, "traffic": None, "kernel": "whole layer"}
    # the whole layer (route .. combine) against the same peak as the dominant kernel
    roof["layer_frac"] = layer_mfma_frac if roof["bound"] == "mfma" else layer_hbm_frac
    if fmt != "int8":
        block_m = splits = None   # chosen inside the layer call by that format's own plan
    return {"T": T, "value": T / (ms_per_step / 1e3), "ms_per_step": ms_per_step,
            "ms_per_step_median": float(np.median(step_ms)), "wall_s": wall,
            "block_m": block_m, "splits": splits, "active_experts": n_active, "flush_mb": flush_mb,
            "bytes": bytes_layer, "flops": flops_layer, "hbm_frac": layer_hbm_frac, "mfma_frac": layer_mfma_frac,
            "stage_ms": stage_ms, "roofline": roof, "xb": xb, "logits_np": logits_np, "active": active}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this library runs on a "
              f"single GPU (the layer is data-parallel over tokens, with no exchange between GPUs).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import weight_quantized_mixture_amd as pkg
    from weight_quantized_mixture_amd import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return
    wl = synthetic.WORKLOADS[args.workload]
    T = args.tokens or HEADLINE_T[args.workload]
    E, k, H, I = wl.E, wl.k, wl.H, wl.I
    w4 = wl.weights == "w4"
    fmt = args.weights
    if w4 and fmt != "int8":
        print(f"--weights {fmt} applies to the int8 workloads; {wl.name} is the uint4 workload",
              file=sys.stderr, flush=True)
        sys.exit(2)

    # ---- set-up: seeded weights quantized on the GPU (not part of a step) ----------
    t0 = time.time()
    if w4:
        layer = pkg.W4A16MoE(E, H, I, wl.group_size, device=dev)
    elif fmt == "fp8":
        layer = pkg.WFP8A16MoE(E, H, I, device=dev)
    else:
        layer = pkg.W8A16MoE(E, H, I, device=dev)
    for e in range(E):
        m13 = torch.from_numpy(synthetic.expert_master(wl, "w13", e, args.seed)).to(dev)
        m2 = torch.from_numpy(synthetic.expert_master(wl, "w2", e, args.seed)).to(dev)
        layer.load_expert(e, m13, m2)
        del m13, m2
    torch.cuda.synchronize()
    log(f"[bench] weights ready ({time.time() - t0:.1f}s) workload={wl.name} T={T}")

    m = measure(pkg, synthetic, torch, dev, layer, wl, T, args, fmt=fmt)
    log(f"[bench] {wl.name} T={T}: {m['ms_per_step'] * 1e3:.1f} us/step")

    # ---- the metric's other band: Mixtral prefill T=4096 on the same weights -----------
    prefill = None
    if wl.name == "mixtral_decode" and not args.no_prefill_band:
        pwl = synthetic.WORKLOADS["mixtral_prefill"]
        pm = measure(pkg, synthetic, torch, dev, layer, pwl, PREFILL_BAND_T, args, fmt=fmt)
        log(f"[bench] {pwl.name} T={PREFILL_BAND_T}: {pm['ms_per_step'] * 1e3:.1f} us/step")
        r = pm["roofline"]
        prefill = {"workload": pwl.name, "T": PREFILL_BAND_T, "value": pm["value"], "steps": args.steps,
                   "ms_per_step": pm["ms_per_step"], "mfma_frac": pm["mfma_frac"],
                   "roofline": {"kernel": r["kernel"], "frac": r["frac"], "kernel_ms": r.get("kernel_ms"),
                                "traffic": r["traffic"]}}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T, m["xb"], m["logits_np"], args, m["active"], fmt)

    res = {
        "metric": "MoE-layer tokens/s",
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int8" if fmt == "w8a8" else
                 ("fp16" if wl.act == "fp16" else "bf16") + (" x uint4" if w4 else " x fp8e4m3" if fmt == "fp8"
                                                            else " x int8"),
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "E": E, "top_k": k, "H": H, "I": I,
                   "weights": "uint4 g128 asym" if w4 else {"int8": "int8 per-channel sym",
                                                             "fp8": "fp8 e4m3fn per-tensor",
                                                             "w8a8": "int8 per-channel sym, int8 per-token act"}[fmt],
                   "block_m": m["block_m"], "splits": m["splits"], "active_experts": m["active_experts"],
                   "flush_mb_between_steps": m["flush_mb"]},
        "stage_ms": m["stage_ms"],
        "layer": {"hbm_frac": m["hbm_frac"], "mfma_frac": m["mfma_frac"]},
        "prefill": prefill,
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
    }
    # compact: the whole line has to survive in a short log tail
    print(json.dumps(_rnd(res, 4), separators=(",", ":")), flush=True)


def gemm1_kernel_name(block_m, H):
    """Name prefix of the GEMM1 kernel the library launches for this block size."""
    if block_m == 256:
        return "gemm1_big_kernel"
    if block_m in (16, 32):
        return "gemm1_dma_kernel"
    if block_m == 64:
        return "gemm1_lds_kernel"
    if block_m == 48:
        return "gemm1_stream_kernel"
    return "gemm1_w8_kernel"


def cpu_baseline(wl, T, xb, logits_np, args, active, fmt="int8"):
    """The fp64 oracle (as it stands) on the host cores: routing + quantized-expert forward."""
    import oracle
    from weight_quantized_mixture_amd import synthetic

    threads, blas = host_blas()
    # the W8A8 oracle sums in int64 numpy matmuls (no BLAS): a smaller sample keeps it to seconds
    Ts = args.cpu_sample_tokens or min(T, 16 if fmt == "w8a8" else 64)
    rows = np.linspace(0, T - 1, Ts).astype(int)
    w_ref, ids_ref = oracle.route_softmax_topk(logits_np[rows], wl.k, wl.renormalize)
    used = np.unique(ids_ref)
    # the oracle quantizes its own weights (not timed: offline in the method too)
    t0 = time.time()
    if wl.weights == "w8" and fmt != "int8":
        # the format's own oracle forward over full-shape parameters (experts the sample never
        # routes to stay zero)
        E, H, I = wl.E, wl.H, wl.I
        q_dt = np.uint8 if fmt == "fp8" else np.int8
        q13 = np.zeros((E, 2 * I, H), q_dt)
        q2 = np.zeros((E, H, I), q_dt)
        s13 = np.zeros(E if fmt == "fp8" else (E, 2 * I), np.float32)
        s2 = np.zeros(E if fmt == "fp8" else (E, H), np.float32)
        quant = oracle.quantize_fp8_tensor if fmt == "fp8" else oracle.quantize_int8_rows
        for e in used:
            q13[e], s13[e] = quant(synthetic.expert_master(wl, "w13", e, args.seed))
            q2[e], s2[e] = quant(synthetic.expert_master(wl, "w2", e, args.seed))
        forward = oracle.moe_forward_fp8 if fmt == "fp8" else oracle.moe_forward_w8a8
        log(f"[bench] oracle weights ready ({time.time() - t0:.1f}s)")
        x = oracle.act_bits_to_f64(xb[rows], wl.act)
        t1 = time.perf_counter()
        w_ref, ids_ref = oracle.route_softmax_topk(logits_np[rows], wl.k, wl.renormalize)
        forward(x, q13, s13, q2, s2, w_ref, ids_ref)
        dt = time.perf_counter() - t1
        return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                "seconds": round(dt, 3), "cpu": host_cpu_model(), "blas": blas,
                "sample": f"{Ts}/{T} tokens: route + {fmt} oracle forward over {used.size} experts"}
    if wl.weights == "w8":
        q13 = {}; s13 = {}; q2 = {}; s2 = {}
        for e in used:
            q13[e], s13[e] = oracle.quantize_int8_rows(synthetic.expert_master(wl, "w13", e, args.seed))
            q2[e], s2[e] = oracle.quantize_int8_rows(synthetic.expert_master(wl, "w2", e, args.seed))
        w13_of = lambda e: oracle.dequant_int8_rows(q13[e], s13[e])  # noqa: E731
        w2_of = lambda e: oracle.dequant_int8_rows(q2[e], s2[e])  # noqa: E731
    else:
        g = wl.group_size
        P = {}
        for e in used:
            q, s, z = oracle.quantize_w4_groups(synthetic.expert_master(wl, "w13", e, args.seed), g)
            q2_, s2_, z2_ = oracle.quantize_w4_groups(synthetic.expert_master(wl, "w2", e, args.seed), g)
            P[e] = (oracle.pack_w4_along_k(q), s, oracle.pack_w4_along_n(z),
                    oracle.pack_w4_along_k(q2_), s2_, oracle.pack_w4_along_n(z2_))
        w13_of = lambda e: oracle.dequant_w4(P[e][0], P[e][1], P[e][2], g)  # noqa: E731
        w2_of = lambda e: oracle.dequant_w4(P[e][3], P[e][4], P[e][5], g)  # noqa: E731
    log(f"[bench] oracle weights ready ({time.time() - t0:.1f}s)")
    x = oracle.act_bits_to_f64(xb[rows], wl.act)
    t1 = time.perf_counter()
    w_ref, ids_ref = oracle.route_softmax_topk(logits_np[rows], wl.k, wl.renormalize)
    oracle.moe_forward_dense(x, w13_of, w2_of, w_ref, ids_ref, wl.I)
    dt = time.perf_counter() - t1
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "cpu": host_cpu_model(), "blas": blas,
            "sample": f"{Ts}/{T} tokens: route + fp64 forward, dequant of {used.size} experts"}


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_blas():
    """(threads, 'vendor version') of the BLAS numpy uses, from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            p = libs[0]
            return int(p.get("num_threads", 1)), f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


if __name__ == "__main__":
    main()
