"""Benchmark of the blockwise W8A8 FP8 hot path on one MI355X.

One step = the linear-layer forward of one Qwen3-8B-shaped layer at prefill
(M = 8192 tokens, activations N(0,1) with 1% outlier channels x30): quantize
the four BF16 activations (qkv 4096, o 4096, gate_up 4096, down 12288 input
features) per token in 1x128 groups, and run the four block-scaled FP8
GEMMs (qkv 4096->6144, o 4096->4096, gate_up 4096->24576, down
12288->4096; FP32 accumulation, BF16 output) on E4M3 weights with
128x128-block scales quantized beforehand (once per RL step).  Both
operands' codes are in the MFMA fragment order that the library's fastest
GEMM reads (quantize_weights_blockwise_frag_multi,
quantize_act_per_token_group_frag, gemm_w8a8_blockscaled_frag: its path for
M % 16 == 0, N % 16 == 0 and K % 256 == 0).
Steps cycle through four copies of every buffer (1.4 GB each), so a copy
has left the 256 MB Infinity Cache before it is used again.  Inputs are
seeded synthetic tensors already resident in HBM.

`value` = GEMM FLOPs of the step / step time (TFLOP/s, the activation
quantization inside the timed step).  The same run measures the per-step
weight re-quantization of all 36 layers of the model (6.95 G parameters,
20.84 GB algorithmic traffic; `requant_GBps`, `roofline_per_kernel.requant`),
checks sampled outputs of both against the CPU oracle (`parity`), times the
oracle on the host's cores (`cpu_baseline`), and adds per-configuration
measurements (`detail`: the decode layer step at M = 256, the prefill
GEMMs on the three operand layouts, the Qwen3-30B-A3B MoE layer, and the
widened operations).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-detail] [--no-cpu]
       python bench.py --rocprof-summary DIR      summarise rocprofv3 runs of this benchmark
       python bench.py --gemm-profile | --gemm-counter-summary DIR
       python bench.py --bw-profile | --bw-counter-summary DIR

`roofline.traffic` is the HBM traffic per launch of the dominant kernel as
measured by rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, scaled by what
the same counters read for a plain copy of known size).  bench.py takes it
from the committed profile summary under profiles/ when that summary was
taken on the current kernel sources (same SHA-256), and reports null
otherwise.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "fp8_blockwise_quantized_quantize_amd", "csrc")
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "prefill_layer_step_qwen3_8b.md")

PREFILL_M = 8192
OUTLIER_FRAC, OUTLIER_MULT = 0.01, 30.0
SWEEP_LAYERS = 36
SWEEP_REPS = 20
# kernel-name prefix and source file of each measured phase; launches per
# step (headline phases) or per sweep (requant: four calls with batch = 36)
PHASE_KERNELS = {
    "act_quant": ("quant_act_frag_kernel", "quant.hip"),
    "gemm": ("gemm_dense_kernel", "gemm.hip"),
    "requant": ("quant_weight_kernel", "quant.hip"),
}
PHASE_LAUNCHES = {"act_quant": 4, "gemm": 4, "requant": 4}


def _code_only(text):
    """C++ source with its comments removed and whitespace runs collapsed
    (what the compiler sees; the kernel sources hold no string literal
    that contains a comment marker)."""
    text = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    return " ".join(text.split())


def source_sha(fname):
    """SHA-256 of a kernel source plus every shared device header, comments
    and whitespace aside (editing a comment does not change the kernel the
    counters were taken on)."""
    h = hashlib.sha256()
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".hpp"))
    for f in (fname, *headers):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(phase):
    """Measured HBM bytes per launch for `phase` from the committed profile
    summary, or None when it is missing or was taken on other sources."""
    try:
        text = open(PROFILE_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"^traffic-json: (\{.*\})$", text, flags=re.M)
    if not m:
        return None
    entry = json.loads(m.group(1)).get(phase)
    if not entry or entry.get("source_sha") != source_sha(PHASE_KERNELS[phase][1]):
        return None
    return entry


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-detail", action="store_true", help="skip the per-configuration measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity check")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale HBM byte counters) and exit")
    p.add_argument("--rocprof-summary", metavar="DIR",
                   help="summarise rocprofv3 output under DIR (kernel trace + FETCH_SIZE / WRITE_SIZE passes "
                        "of this benchmark and of --calibrate-copy) and exit")
    p.add_argument("--gemm-profile", action="store_true",
                   help="only run each GEMM of gemm_profile_cases() a few times (a target for rocprofv3 "
                        "counter passes) and exit")
    p.add_argument("--gemm-counter-summary", metavar="DIR",
                   help="summarise rocprofv3 passes of --gemm-profile under DIR (kt, mfma, lds, l2, fetch, "
                        "write, copy_fetch, copy_write) and exit")
    p.add_argument("--bw-profile", action="store_true",
                   help="only run each bandwidth-bound kernel of bw_profile_cases() a few times (a target for "
                        "FETCH_SIZE / WRITE_SIZE passes) and exit")
    p.add_argument("--bw-counter-summary", metavar="DIR",
                   help="summarise rocprofv3 passes of --bw-profile under DIR (kt, fetch, write, copy_fetch, "
                        "copy_write) and exit")
    return p.parse_args()


def device_info():
    """GPU name and architecture, CU count and the HIP / torch versions of the run."""
    import torch

    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__}


def calibrate_copy():
    """A plain device-to-device copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def host_threads():
    """Worker threads for the CPU oracle: the host cores this process may
    use, at most 16 (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.gemm_profile:
        gemm_profile()
        return
    if args.gemm_counter_summary:
        gemm_counter_summary(args.gemm_counter_summary)
        return
    if args.bw_profile:
        bw_profile()
        return
    if args.bw_counter_summary:
        bw_counter_summary(args.bw_counter_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path.  Its kernels run on "
              "one GPU's share of the work: whole 128x128 weight blocks for re-quantization, column- or "
              "row-parallel GEMM slices at multiples of 128, or whole experts.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, ROOT)
    import fp8_blockwise_quantized_quantize_amd as fb
    from synthetic import LAYER_SHAPES_QWEN3_8B, device_activations, device_bf16_normal

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    M = PREFILL_M

    # ---------------------------------------------------------------- inputs
    # Step s uses buffer set s % SETS (copies of the same inputs, 1.4 GB per
    # set): a set's bytes have left the 256 MB Infinity Cache before it is
    # used again.  The weights are quantized once, before the timed steps,
    # into the MFMA fragment order the GEMM reads (as the per-step
    # re-quantization writes them).
    SETS = 4
    base = []
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((n, k), 0.02, seed=300 + i)
        x, _ = device_activations(M, k, seed=400 + 2 * i, outlier_frac=OUTLIER_FRAC, outlier_mult=OUTLIER_MULT)
        base.append((name, n, k, w, x))
    sets = []
    for c in range(SETS):
        layers = []
        for name, n, k, w, x in base:
            layers.append({
                "name": name, "n": n, "k": k, "x": x if c == 0 else x.clone(),
                "wq": torch.empty((n, k), dtype=torch.uint8, device=dev),
                "ws": torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev),
                "xq": torch.empty((M, k), dtype=torch.uint8, device=dev),
                "xs": torch.empty((M, k // 128), dtype=torch.float32, device=dev),
                "y": torch.empty((M, n), dtype=torch.bfloat16, device=dev),
            })
        fb.quantize_weights_blockwise_frag_multi([b[3] for b in base], [(L["wq"], L["ws"]) for L in layers])
        sets.append(layers)
    w_bf16 = {name: w for name, _, _, w, _ in base}
    del base
    layers = sets[0]
    gemm_flops = sum(2 * M * L["n"] * L["k"] for L in layers)
    act_bytes = sum(M * L["k"] * 3 + M * (L["k"] // 128) * 4 for L in layers)
    gemm_bytes = sum(M * L["k"] + L["n"] * L["k"] + 2 * M * L["n"] + M * (L["k"] // 128) * 4
                     + (L["n"] // 128) * (L["k"] // 128) * 4 for L in layers)

    # HIP events between the two phases of a step, on the launch stream
    phases = ("act_quant", "gemm")
    ev = []

    def step(record, s):
        ls = sets[s % SETS]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if record else None
        if record:
            e[0].record(stream)
        for L in ls:
            fb.quantize_act_per_token_group_frag(L["x"], L["xq"], L["xs"])
        if record:
            e[1].record(stream)
        for L in ls:
            fb.gemm_w8a8_blockscaled_frag(L["xq"], L["xs"], L["wq"], L["ws"], L["y"])
        if record:
            e[2].record(stream)
            ev.append(e)

    for s in range(args.warmup):
        step(False, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(True, s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12
    step(False, 0)  # set 0 holds this step's outputs for the parity check
    torch.cuda.synchronize()
    phase_ms = {p: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / len(ev) for i, p in enumerate(phases)}

    # ------------------------------------------- the 36-layer re-quant sweep
    sweep = requant_sweep(fb, dev)

    roof_all = {
        "gemm": roof_entry("gemm", phase_ms["gemm"], gemm_bytes, gemm_flops),
        "act_quant": roof_entry("act_quant", phase_ms["act_quant"], act_bytes, 0),
        "requant": roof_entry("requant", sweep["ms"], sweep["bytes"], 0),
    }
    roof_all["requant"].update({"reps": sweep["reps"], "median_ms": sweep["median_ms"], "min_ms": sweep["min_ms"]})
    dominant = max(phases, key=lambda p: phase_ms[p])
    roofline = dict(roof_all[dominant])

    out = {
        "metric": "W8A8 block-scaled GEMM TFLOP/s + weight re-quant GB/s (% of roofline)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded N(0,0.02) weights; N(0,1) activations with 1% outlier channels x30; "
                "Qwen3-8B layer shapes; 4 buffer sets rotated across steps)",
        "config": {
            "workload": "qwen3-8b-prefill-layer: 1x128 act quant + 4 W8A8 block-scaled GEMMs "
                        "(qkv/o/gate_up/down), M=8192, operands in MFMA fragment order",
            "tokens": M,
            "gemm_flops_per_step": gemm_flops,
            "requant_workload": "qwen3-8b 36-layer weight re-quant sweep: 6.95 G params, 4 calls with batch=36, "
                                "codes in fragment order",
            "parallelism": "1 GPU",
        },
        "roofline": roofline,
        "roofline_per_kernel": roof_all,
        "phase_ms": {p: round(v, 4) for p, v in phase_ms.items()},
        "requant_GBps": roof_all["requant"]["achieved"],
        "requant_frac_hbm": roof_all["requant"]["frac"],
        "device": device_info(),
    }

    if not args.no_cpu:
        out["cpu_baseline"], out["parity"] = cpu_baseline_and_parity(fb, layers, w_bf16, sweep, gemm_flops)
    sweep.pop("tensors")
    torch.cuda.empty_cache()
    if not args.no_detail:
        out["detail"] = detail(fb, dev, with_cpu=not args.no_cpu)
        legs = {name: leg["parity"]["pass"] for name, leg in out["detail"].items()
                if isinstance(leg, dict) and isinstance(leg.get("parity"), dict) and "pass" in leg["parity"]}
        if legs and isinstance(out.get("parity"), dict):
            out["parity"]["detail"] = legs
            out["parity"]["pass"] = bool(out["parity"].get("pass", True) and all(legs.values()))
    print(json.dumps(out), flush=True)


def roof_entry(phase, ms, byt, flops):
    """Roofline of one measured phase: the FP8 MFMA peak when its arithmetic
    intensity passes the ridge point, HBM bandwidth otherwise."""
    name = PHASE_KERNELS[phase][0]
    nl = PHASE_LAUNCHES[phase]
    if flops and flops / byt > FP8_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3:
        ach, peak, unit, bound = flops / ms / 1e9, FP8_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = byt / ms / 1e6, HBM_PEAK_GBPS, "GB/s", "hbm"
    tr = committed_traffic(phase)
    e = {"bound": bound, "kernel": name, "achieved": round(ach, 1), "peak": peak, "unit": unit,
         "frac": round(ach / peak, 4), "traffic": tr["bytes_per_launch"] if tr else None,
         "avg_launch_us": round(ms * 1e3 / nl, 2), "launches": nl,
         "algorithmic_bytes_per_launch_avg": int(byt / nl), "flops_per_launch_avg": int(flops / nl)}
    if flops:
        e["TFLOPs"] = round(flops / ms / 1e9, 1)
    return e


def requant_sweep(fb, dev, frag=True):
    """The per-step re-quantization of every quantized linear weight of the
    model: 36 layers x {qkv, o, gate_up, down} (6.95 G BF16 parameters),
    four calls with batch = 36, codes in fragment order (frag) or row-major.
    SWEEP_REPS timed sweeps (HIP events around each) after two untimed ones;
    21 GB per sweep, far past the Infinity Cache, so no rotation is needed."""
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, device_bf16_normal

    bufs, byt = [], 0
    for p, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((SWEEP_LAYERS, n, k), 0.02, seed=800 + p)
        q = torch.empty((SWEEP_LAYERS, n, k), dtype=torch.uint8, device=dev)
        s = torch.empty((SWEEP_LAYERS, n // 128, k // 128), dtype=torch.float32, device=dev)
        bufs.append((name, w, q, s))
        byt += SWEEP_LAYERS * n * k * 3 + s.numel() * 4

    def run():
        for _, w, q, s in bufs:
            fb.quantize_weight_blockwise(w, q, s, frag=frag)

    for _ in range(2):
        run()
    st = torch.cuda.current_stream()
    evs = []
    for _ in range(SWEEP_REPS):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        run()
        b.record(st)
        evs.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return {"ms": sum(t) / len(t), "median_ms": t[len(t) // 2], "min_ms": t[0], "reps": len(t), "bytes": byt,
            "params": sum(w.numel() for _, w, _, _ in bufs), "frag": frag, "tensors": bufs}


# ---------------------------------------------------------------------------
# Timing helpers for the per-configuration measurements
# ---------------------------------------------------------------------------

def _time_ms(fn, reps, warm=2):
    """Median per-call time with HIP events on the current stream."""
    import torch

    for _ in range(warm):
        fn()
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        times.append((a, b))
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) for a, b in times)
    return v[len(v) // 2], v[0]


ROTATE_BYTES = 1 << 30  # a rotation of buffer sets larger than the 256 MB Infinity Cache


def rotations(bytes_per_set, cap=16):
    """Buffer sets to cycle through so that a call's working set has left the
    256 MB Infinity Cache before the same set comes round again."""
    return max(1, min(cap, -(-ROTATE_BYTES // max(1, bytes_per_set))))


def _time_graph_ms(fn, calls=10, reps=5):
    """Median GPU time per call, from replays of a HIP graph holding `calls`
    back-to-back calls (host call overhead excluded: small kernels would
    otherwise be timed at the speed of their Python wrapper).  `fn` is one
    callable or a list of callables on different buffer sets, used in turn.
    Falls back to per-call events when the calls cannot be captured."""
    import torch

    fns = fn if isinstance(fn, (list, tuple)) else [fn]
    calls = max(calls, len(fns))
    try:
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(calls):
                    fns[i % len(fns)]()
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) / calls)
        times.sort()
        return times[len(times) // 2], times[0]
    except RuntimeError:
        return _time_ms(fns[0], reps=10)


# ---------------------------------------------------------------------------
# Per-configuration measurements (after the timed region)
# ---------------------------------------------------------------------------

def detail(fb, dev, with_cpu=True):
    import torch

    res = {}
    # -- the Qwen3-8B decode layer step (M = 256): re-quantize the layer's four
    #    weights, quantize its four activations, four GEMMs
    res["decode_layer_qwen3_8b_M256"] = decode_step(fb, dev, with_cpu)
    torch.cuda.empty_cache()
    # -- prefill GEMMs one by one, both activation layouts, rotated buffers
    res["prefill_gemm_M8192"] = prefill_gemms(fb, dev)
    torch.cuda.empty_cache()
    # -- one MoE expert-FFN layer (Qwen3-30B-A3B: 4096 tokens, top-8 of 128
    #    experts, hidden 2048, expert FFN 768), every step on the GPU
    res["moe_layer_qwen3_30b_a3b"] = moe_layer(fb, dev, with_cpu)
    torch.cuda.empty_cache()
    # -- FP8 training operands (Qwen3-8B)
    res["train_operands_qwen3_8b"] = train_operands(fb, dev, with_cpu)
    torch.cuda.empty_cache()
    # -- FP8 KV cache, one Qwen3-8B layer (8 KV heads x 128)
    res["kv_cache_qwen3_8b_layer"] = kv_cache(fb, dev, with_cpu)
    torch.cuda.empty_cache()
    # -- token-level TIS weights of one training batch (512 responses padded
    #    to 20,000 tokens), fused with the response mask and w * advantage
    res["tis_weights_train_batch_512x20000"] = tis_weights(fb, dev, with_cpu)
    torch.cuda.empty_cache()
    return res


def decode_step(fb, dev, with_cpu):
    """The Qwen3-8B decode layer step at M = 256: one launch re-quantizes the
    four weight matrices, one launch quantizes the four activations (codes
    of both in fragment order), then the four fragment-order GEMMs.  Steps cycle
    through four copies of the layer's buffers (0.6 GB each).  Phases timed
    with HIP events; the oracle runs the same step on the same input bytes
    (parity and a CPU time on all its threads)."""
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, device_bf16_normal

    M, SETS, STEPS, WARM = 256, 4, 50, 5
    sets = []
    for c in range(SETS):
        layers = []
        for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
            w = device_bf16_normal((n, k), 0.02, seed=100 + i) if c == 0 else sets[0][i]["w"].clone()
            x = device_bf16_normal((M, k), 1.0, seed=200 + i) if c == 0 else sets[0][i]["x"].clone()
            layers.append({
                "name": name, "n": n, "k": k, "w": w, "x": x,
                "wq": torch.empty((n, k), dtype=torch.uint8, device=dev),
                "ws": torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev),
                "xq": torch.empty((M, k), dtype=torch.uint8, device=dev),
                "xs": torch.empty((M, k // 128), dtype=torch.float32, device=dev),
                "y": torch.empty((M, n), dtype=torch.bfloat16, device=dev),
            })
        sets.append(layers)
    stream = torch.cuda.current_stream()
    ev = []

    def step(record, s):
        ls = sets[s % SETS]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        fb.quantize_weights_blockwise_frag_multi([L["w"] for L in ls], [(L["wq"], L["ws"]) for L in ls])
        if record:
            e[1].record(stream)
        fb.quantize_acts_per_token_group_frag_multi([L["x"] for L in ls], [(L["xq"], L["xs"]) for L in ls])
        if record:
            e[2].record(stream)
        for L in ls:
            fb.gemm_w8a8_blockscaled_frag(L["xq"], L["xs"], L["wq"], L["ws"], L["y"])
        if record:
            e[3].record(stream)
            ev.append(e)

    for s in range(WARM):
        step(False, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(STEPS):
        step(True, s)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / STEPS
    step(False, 0)
    torch.cuda.synchronize()
    layers = sets[0]
    flops = sum(2 * M * L["n"] * L["k"] for L in layers)
    rq_b = sum(L["n"] * L["k"] * 3 + L["ws"].numel() * 4 for L in layers)
    aq_b = sum(M * L["k"] * 3 + L["xs"].numel() * 4 for L in layers)
    gm_b = sum(M * L["k"] + L["n"] * L["k"] + 2 * M * L["n"] + L["xs"].numel() * 4 + L["ws"].numel() * 4
               for L in layers)
    ph = {p: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / len(ev)
          for i, p in enumerate(("requant", "act_quant", "gemm"))}
    res = {"ms_per_step": round(ms, 4), "TFLOPs": round(flops / ms / 1e9, 1), "steps": STEPS, "buffer_sets": SETS,
           "phase_us": {p: round(v * 1e3, 2) for p, v in ph.items()},
           "requant": {"launches": 1, "bytes": rq_b, "GBps": round(rq_b / ph["requant"] / 1e6, 1),
                       "frac_hbm": round(rq_b / ph["requant"] / 1e6 / HBM_PEAK_GBPS, 4)},
           "act_quant": {"launches": 1, "bytes": aq_b, "GBps": round(aq_b / ph["act_quant"] / 1e6, 1)},
           "gemm": {"launches": 4, "bytes": gm_b, "TFLOPs": round(flops / ph["gemm"] / 1e9, 1),
                    "GBps": round(gm_b / ph["gemm"] / 1e6, 1),
                    "frac_hbm": round(gm_b / ph["gemm"] / 1e6 / HBM_PEAK_GBPS, 4)}}
    # each GEMM on its own, as the step runs it (graph replays over the four
    # buffer sets), and on the other operand layouts: fragment-order
    # activations with row-major weights, and both row-major
    for ls in sets:
        for L in ls:
            L["xr"], _ = fb.quantize_act_per_token_group(L["x"])
            L["wr"], _ = fb.quantize_weight_blockwise(L["w"])
    per = {}
    for i, L in enumerate(layers):
        f = 2 * M * L["n"] * L["k"]
        byt = M * L["k"] + L["n"] * L["k"] + 2 * M * L["n"] + L["xs"].numel() * 4 + L["ws"].numel() * 4
        us, _ = _time_graph_ms([lambda t=t[i]: fb.gemm_w8a8_blockscaled_frag(t["xq"], t["xs"], t["wq"], t["ws"],
                                                                             t["y"]) for t in sets])
        y_frag = layers[i]["y"].clone()
        af, _ = _time_graph_ms([lambda t=t[i]: fb.gemm_w8a8_blockscaled_afrag(t["xq"], t["xs"], t["wr"], t["ws"],
                                                                              t["y"]) for t in sets])
        y_afrag = layers[i]["y"].clone()
        rm, _ = _time_graph_ms([lambda t=t[i]: fb.gemm_w8a8_blockscaled(t["xr"], t["xs"], t["wr"], t["ws"], t["y"])
                                for t in sets])
        y_row = layers[i]["y"]
        same = torch.equal(y_frag.view(torch.int16), y_row.view(torch.int16)) and torch.equal(
            y_afrag.view(torch.int16), y_row.view(torch.int16))
        per[L["name"]] = {"us": round(us * 1e3, 2), "frac_hbm": round(byt / us / 1e6 / HBM_PEAK_GBPS, 4),
                          "TFLOPs": round(f / us / 1e9, 1), "afrag_us": round(af * 1e3, 2),
                          "row_major_us": round(rm * 1e3, 2), "bit_identical": bool(same)}
    res["gemm_each"] = per
    res["splitk_small_batch"] = splitk_small_batch(fb, dev, sets[0])
    for ls in sets:
        for L in ls:
            del L["xr"], L["wr"]
    step(False, 0)
    torch.cuda.synchronize()
    if with_cpu:
        res["cpu_baseline"], res["parity"] = decode_cpu_and_parity(layers, M, flops)
    return res


def splitk_small_batch(fb, dev, layer_set):
    """The K-split GEMM against the unsplit one at small decode batches
    (16, 64 and 128 tokens) on the Qwen3-8B layer weights, which the split
    rule splits where K is long against M (the down projection): graph
    replays over four weight copies (Infinity Cache rotated)."""
    import torch

    res = {}
    for m in (16, 64, 128):
        for L in layer_set:
            n, k = L["n"], L["k"]
            need = fb.splitk_workspace_bytes(m, n, k)
            if need == 0:
                continue
            wq = [L["wr"]] + [L["wr"].clone() for _ in range(3)]
            xq, xs = L["xr"][:m].contiguous(), L["xs"][:m].contiguous()
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty(need, dtype=torch.uint8, device=dev)
            sk, _ = _time_graph_ms([lambda w=w: fb.gemm_w8a8_blockscaled_splitk(xq, xs, w, L["ws"], y, workspace=wsp)
                                    for w in wq])
            pl, _ = _time_graph_ms([lambda w=w: fb.gemm_w8a8_blockscaled(xq, xs, w, L["ws"], y) for w in wq])
            res["%s_M%d" % (L["name"], m)] = {"k_pieces": need // (4 * m * n), "splitk_us": round(sk * 1e3, 2),
                                               "unsplit_us": round(pl * 1e3, 2)}
    return res


def prefill_gemms(fb, dev):
    """Each prefill GEMM (M = 8192) on its own, on three operand layouts
    (both row-major; fragment-order activations; both in fragment order),
    timed from graph replays over enough buffer copies (input codes,
    weights, output) that a copy has left the Infinity Cache before it comes
    round again; the layouts' outputs compared bit for bit."""
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, device_activations, device_bf16_normal

    m = PREFILL_M
    pre, tot_f = {}, 0.0
    tot = {"row": 0.0, "afrag": 0.0, "frag": 0.0}
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        wb = device_bf16_normal((n, k), 0.02, seed=300 + i)
        wq, ws = fb.quantize_weight_blockwise(wb)
        wf, _ = fb.quantize_weight_blockwise_frag(wb)
        del wb
        x, _ = device_activations(m, k, seed=400 + 2 * i, outlier_frac=OUTLIER_FRAC, outlier_mult=OUTLIER_MULT)
        xq, xs = fb.quantize_act_per_token_group(x)
        xf, _ = fb.quantize_act_per_token_group_frag(x)
        nsets = rotations(2 * m * k + 2 * n * k + 2 * m * n)
        mk = lambda c: {"xq": xq if c == 0 else xq.clone(), "xf": xf if c == 0 else xf.clone(),
                        "xs": xs if c == 0 else xs.clone(), "wq": wq if c == 0 else wq.clone(),
                        "wf": wf if c == 0 else wf.clone(), "ws": ws if c == 0 else ws.clone(),
                        "y": torch.empty((m, n), dtype=torch.bfloat16, device=dev)}
        sets = [mk(c) for c in range(nsets)]
        calls = max(4, nsets)
        ms = {}
        ms["row"], _ = _time_graph_ms([lambda t=t: fb.gemm_w8a8_blockscaled(t["xq"], t["xs"], t["wq"], t["ws"], t["y"])
                                       for t in sets], calls=calls)
        y_row = sets[0]["y"].clone()
        ms["afrag"], _ = _time_graph_ms([lambda t=t: fb.gemm_w8a8_blockscaled_afrag(t["xf"], t["xs"], t["wq"], t["ws"],
                                                                                    t["y"]) for t in sets], calls=calls)
        same = torch.equal(y_row.view(torch.int16), sets[0]["y"].view(torch.int16))
        ms["frag"], _ = _time_graph_ms([lambda t=t: fb.gemm_w8a8_blockscaled_frag(t["xf"], t["xs"], t["wf"], t["ws"],
                                                                                  t["y"]) for t in sets], calls=calls)
        same = same and torch.equal(y_row.view(torch.int16), sets[0]["y"].view(torch.int16))
        del sets, y_row
        xsets = [(x, torch.empty_like(xq), torch.empty_like(xs))]
        xsets += [(x.clone(), torch.empty_like(xq), torch.empty_like(xs)) for _ in range(rotations(m * k * 3) - 1)]
        aq_ms, _ = _time_graph_ms([lambda t=t: fb.quantize_act_per_token_group(*t) for t in xsets])
        aqf_ms, _ = _time_graph_ms([lambda t=t: fb.quantize_act_per_token_group_frag(*t) for t in xsets])
        del xsets
        f = 2 * m * n * k
        tot_f += f
        for key in tot:
            tot[key] += ms[key]
        aq_b = m * k * 3 + m * (k // 128) * 4
        e = {"buffer_sets": nsets, "bit_identical": bool(same)}
        for key, label in (("row", ""), ("afrag", "afrag_"), ("frag", "frag_")):
            e[label + "gemm_us"] = round(ms[key] * 1e3, 1)
            e[label + "TFLOPs"] = round(f / ms[key] / 1e9, 1)
            e[label + "frac_fp8_peak"] = round(f / ms[key] / 1e9 / FP8_PEAK_TFLOPS, 4)
        e.update({"act_quant_us": round(aq_ms * 1e3, 1), "afrag_act_quant_us": round(aqf_ms * 1e3, 1),
                  "act_quant_GBps": round(aq_b / aq_ms / 1e6, 1),
                  "afrag_act_quant_GBps": round(aq_b / aqf_ms / 1e6, 1)})
        pre[name] = e
        del wq, wf, ws, x, xq, xs, xf
        torch.cuda.empty_cache()
    pre["all4"] = {}
    for key, label in (("row", ""), ("afrag", "afrag_"), ("frag", "frag_")):
        pre["all4"][label + "TFLOPs"] = round(tot_f / tot[key] / 1e9, 1)
        pre["all4"][label + "frac_fp8_peak"] = round(tot_f / tot[key] / 1e9 / FP8_PEAK_TFLOPS, 4)
    # the three layouts' outputs, bit for bit (the fragment-order form is the
    # headline's, whose outputs the headline parity checks against the oracle)
    same = all(e["bit_identical"] for nm, e in pre.items() if nm != "all4")
    pre["parity"] = {"layouts_bit_identical": same, "pass": same}
    return pre


def moe_layer(fb, dev, with_cpu=True):
    import torch

    from synthetic import MOE_QWEN3_30B_A3B, device_bf16_normal, moe_topk

    cfg = MOE_QWEN3_30B_A3B
    T, E, k, H, F = cfg["tokens"], cfg["experts"], cfg["top_k"], cfg["hidden"], cfg["ffn"]
    R = T * k
    ids_h, tw_h = moe_topk(T, E, k, (70, 0))
    ids, tw = torch.from_numpy(ids_h).to(dev), torch.from_numpy(tw_h).to(dev)
    x = device_bf16_normal((T, H), 1.0, seed=700)
    w1 = device_bf16_normal((E, 2 * F, H), 0.02, seed=600)
    w2 = device_bf16_normal((E, H, F), 0.02, seed=601)
    # the per-step re-quantization of every expert weight: both stacks in one launch
    w1f, w2f = w1.view(E * 2 * F, H), w2.view(E * H, F)
    (w1q, w1s), (w2q, w2s) = fb.quantize_weights_blockwise_multi([w1f, w2f])
    req_out = [(w1q, w1s), (w2q, w2s)]
    w1q, w1s = w1q.view(E, 2 * F, H), w1s.view(E, 2 * F // 128, H // 128)
    w2q, w2s = w2q.view(E, H, F), w2s.view(E, H // 128, F // 128)
    off, sp, pr = fb.moe_sort_by_expert(ids, E)
    a, a_s = fb.quantize_act_per_token_group(x)
    y1 = torch.empty((R, 2 * F), dtype=torch.bfloat16, device=dev)
    h, h_s = torch.empty((R, F), dtype=torch.uint8, device=dev), torch.empty((R, F // 128), dtype=torch.float32,
                                                                               device=dev)
    y2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    # Each step cycles through copies of its inputs and outputs sized so that
    # a copy has left the 256 MB Infinity Cache before it is used again.
    fb.grouped_gemm_w8a8_blockscaled_gather(a, a_s, sp, k, w1q, w1s, off, y1)
    fb.silu_mul_quantize_act(y1, h, h_s)
    fb.grouped_gemm_w8a8_blockscaled(h, h_s, w2q, w2s, off, y2)

    def copies(n, *ts):
        return [ts] + [tuple(t.clone() for t in ts) for _ in range(n - 1)]

    aq_b = T * H * 3 + T * (H // 128) * 4
    silu_b = R * 2 * F * 2 + R * F + R * (F // 128) * 4
    comb_b = R * H * 2 + R * 8 + T * H * 2
    w1_b, w2_b = w1q.numel() + w1s.numel() * 4, w2q.numel() + w2s.numel() * 4
    aq_sets = copies(rotations(aq_b), x, a, a_s)
    w1_sets = copies(rotations(w1_b), w1q, w1s, y1)
    silu_sets = copies(rotations(silu_b), y1, h, h_s)
    w2_sets = copies(rotations(w2_b), w2q, w2s, y2)
    comb_sets = copies(rotations(comb_b), y2, out)
    req_b = (w1.numel() + w2.numel()) * 3 + (w1s.numel() + w2s.numel()) * 4
    steps = {
        "expert_requant": ([lambda: fb.quantize_weights_blockwise_multi([w1f, w2f], req_out)], req_b, None),
        "sort": ([lambda: fb.moe_sort_by_expert(ids, E, off, sp, pr)], None, None),
        "act_quant": ([lambda t=t: fb.quantize_act_per_token_group(*t) for t in aq_sets], aq_b, None),
        "fc1_gate_up": ([lambda t=t: fb.grouped_gemm_w8a8_blockscaled_gather(a, a_s, sp, k, t[0], t[1], off, t[2])
                         for t in w1_sets], None, 2 * R * 2 * F * H),
        "silu_mul_quant": ([lambda t=t: fb.silu_mul_quantize_act(*t) for t in silu_sets], silu_b, None),
        "fc2_down": ([lambda t=t: fb.grouped_gemm_w8a8_blockscaled(h, h_s, t[0], t[1], off, t[2]) for t in w2_sets],
                     None, 2 * R * H * F),
        "combine": ([lambda t=t: fb.moe_combine(t[0], pr, tw, t[1]) for t in comb_sets], comb_b, None),
    }
    fused_sets = copies(rotations(w1_b), w1q, w1s, h, h_s)
    # fc1 with SiLU(gate) * up quantized in its epilogue: replaces the
    # fc1_gate_up + silu_mul_quant pair (not part of the separate chain's sum).
    steps["fc1_silu_quant_fused"] = ([lambda t=t: fb.grouped_gemm_w8a8_blockscaled_gather_silu(a, a_s, sp, k, t[0], t[1], off,
                                                                                          t[2], t[3])
                                      for t in fused_sets], None, 2 * R * 2 * F * H)
    res, total = {}, 0.0
    for name, (fn, byt, flops) in steps.items():
        ms, _ = _time_graph_ms(fn)
        if name not in ("fc1_silu_quant_fused", "expert_requant"):
            total += ms
        e = {"us": round(ms * 1e3, 1), "buffer_sets": len(fn)}
        if byt is not None:
            e.update({"bytes": byt, "GBps": round(byt / ms / 1e6, 1), "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBPS, 4)})
        if flops is not None:
            fc1 = name.startswith("fc1")
            n_out = 2 * F if fc1 else H
            k_in = H if fc1 else F
            a_rows = T if fc1 else R  # fc1 reads each token's row once (gathered)
            out_b = R * F + R * (F // 128) * 4 if name == "fc1_silu_quant_fused" else 2 * R * n_out
            byt_g = a_rows * k_in + E * n_out * k_in + out_b + a_rows * (k_in // 128) * 4
            roof = min(FP8_PEAK_TFLOPS, flops / byt_g * HBM_PEAK_GBPS / 1e3)
            e.update({"TFLOPs": round(flops / ms / 1e9, 1), "roofline_TFLOPs": round(roof, 1),
                      "frac_roofline": round(flops / ms / 1e9 / roof, 4)})
        res[name] = e

    def layer():
        fb.moe_expert_ffn(x, ids, tw, w1q, w1s, w2q, w2s, fused=True)

    def layer_separate():
        fb.moe_expert_ffn(x, ids, tw, w1q, w1s, w2q, w2s, fused=False)

    layer_ms, _ = _time_graph_ms(layer, calls=4)
    sep_ms, _ = _time_graph_ms(layer_separate, calls=4)
    del aq_sets, w1_sets, silu_sets, w2_sets, comb_sets, fused_sets
    res["sum_of_kernels_us"] = round(total * 1e3, 1)
    res["layer_us"] = round(layer_ms * 1e3, 1)
    res["layer_separate_fc1_silu_us"] = round(sep_ms * 1e3, 1)
    layer_flops = 2 * R * 2 * F * H + 2 * R * H * F
    res["layer_TFLOPs"] = round(layer_flops / layer_ms / 1e9, 1)
    if with_cpu:
        out = fb.moe_expert_ffn(x, ids, tw, w1q, w1s, w2q, w2s)
        hq, hs = fb.grouped_gemm_w8a8_blockscaled_gather_silu(a, a_s, sp, k, w1q, w1s, off)
        y2p = fb.grouped_gemm_w8a8_blockscaled(hq, hs, w2q, w2s, off)
        torch.cuda.synchronize()
        res["cpu_baseline"], res["parity"] = moe_cpu_and_parity(
            x, ids_h, tw_h, w1, w2, w1q, w1s, w2q, w2s, off, sp, pr, out, hq, y2p, layer_flops, req_b)
    return res


def train_operands(fb, dev, with_cpu=True):
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, device_bf16_normal

    res = {}
    bufs = []
    wbytes = 0
    for p, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((36, n, k), 0.02, seed=950 + p)
        bufs.append(w)
        wbytes += 36 * n * k * 4 + 2 * 36 * (n // 128) * (k // 128) * 4

    def sweep():
        for w in bufs:
            fb.quantize_weight_blockwise_dual(w)

    ms, _ = _time_ms(sweep, reps=5, warm=1)
    res["weight_dual_sweep_36_layers"] = {"bytes": wbytes, "ms": round(ms, 3), "GBps": round(wbytes / ms / 1e6, 1),
                                          "frac_hbm": round(wbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
    checks = []  # (label, BF16 input, GPU outputs) for the oracle leg
    if with_cpu:
        for (name, n, k), w in zip(LAYER_SHAPES_QWEN3_8B, bufs):
            (q, sq), (qt, sqt) = fb.quantize_weight_blockwise_dual(w)
            for layer in (35, 0):  # the last layer lies past 2^31 bytes into the batch
                checks.append(("W %s layer %d" % (name, layer), _bits(w[layer]),
                               [t[layer].cpu().numpy() for t in (q, sq, qt, sqt)]))
            del q, sq, qt, sqt
    del bufs
    torch.cuda.empty_cache()
    M = 8192
    for k in (4096, 12288):
        x = device_bf16_normal((M, k), 1.0, seed=960 + k)
        byt = M * k * 4 + M * (k // 128) * 4 + k * (M // 128) * 4
        xs = [x] + [x.clone() for _ in range(rotations(byt) - 1)]
        ms, _ = _time_graph_ms([lambda t=t: fb.quantize_act_dual(t) for t in xs], calls=max(5, len(xs)))
        del xs
        res[f"act_dual_{M}x{k}"] = {"us": round(ms * 1e3, 1), "bytes": byt, "GBps": round(byt / ms / 1e6, 1),
                                    "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        if with_cpu:
            (q, sq), (qt, sqt) = fb.quantize_act_dual(x)
            checks.append(("x %dx%d" % (M, k), _bits(x), [t.cpu().numpy() for t in (q, sq, qt, sqt)]))
        del x
    if with_cpu:
        res["cpu_baseline"], res["parity"] = train_cpu_and_parity(checks)
    return res


def kv_cache(fb, dev, with_cpu=True):
    import torch

    from synthetic import device_bf16_normal

    H, D, T, B = 8, 128, 16384, 1536
    S = T + B
    k = device_bf16_normal((T, H, D), 1.0, seed=900)
    v = device_bf16_normal((T, H, D), 1.0, seed=901)
    kn = device_bf16_normal((B, H, D), 1.0, seed=902)
    vn = device_bf16_normal((B, H, D), 1.0, seed=903)
    ks = torch.empty(H, dtype=torch.float32, device=dev)
    vs = torch.empty(H, dtype=torch.float32, device=dev)
    kc = torch.empty((S, H, D), dtype=torch.uint8, device=dev)
    vc = torch.empty((S, H, D), dtype=torch.uint8, device=dev)
    slots = torch.arange(T, dtype=torch.int32, device=dev)
    dslots = torch.arange(T, S, dtype=torch.int32, device=dev)
    res = {}
    cal_b = 2 * T * H * D * 2
    sets = [(k, v)] + [(k.clone(), v.clone()) for _ in range(rotations(cal_b) - 1)]
    cal_ms, _ = _time_graph_ms([lambda t=t: fb.kv_scale_calibrate(t[0], t[1], True, ks, vs) for t in sets])
    wr_b = 2 * T * H * D * 3 + T * 4
    wsets = [(t[0], t[1], torch.empty_like(kc), torch.empty_like(vc)) for t in sets[:rotations(wr_b)]]
    wr_ms, _ = _time_graph_ms([lambda t=t: fb.kv_cache_write_fp8(t[0], t[1], slots, ks, vs, t[2], t[3])
                               for t in wsets])
    del sets, wsets
    dec_ms, _ = _time_graph_ms(lambda: fb.kv_cache_write_fp8(kn, vn, dslots, ks, vs, kc, vc))
    for name, ms, byt in (("calibrate_16384", cal_ms, cal_b), ("write_16384", wr_ms, wr_b)):
        res[name] = {"us": round(ms * 1e3, 1), "bytes": byt, "GBps": round(byt / ms / 1e6, 1),
                     "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBPS, 4)}
    # 9.4 MB per call: latency-bound, reported in microseconds only
    res["decode_write_1536"] = {"us": round(dec_ms * 1e3, 1), "bytes": 2 * B * H * D * 3 + B * 4}
    if with_cpu:  # one calibration, the prefill write and the decode write, then the oracle
        fb.kv_scale_calibrate(k, v, True, ks, vs)
        fb.kv_cache_write_fp8(k, v, slots, ks, vs, kc, vc)
        fb.kv_cache_write_fp8(kn, vn, dslots, ks, vs, kc, vc)
        torch.cuda.synchronize()
        res["cpu_baseline"], res["parity"] = kv_cpu_and_parity(
            [_bits(t) for t in (k, v, kn, vn)], ks.cpu().numpy(), vs.cpu().numpy(), kc.cpu().numpy(),
            vc.cpu().numpy(), cal_b, wr_b)
    return res


def importance_weight_bytes(slots, valid):
    """Algorithmic HBM bytes of the fused importance-weight pass: the two
    log-probs and the advantage of each generated token (12 B), the mask byte
    and the two float32 outputs of every slot, padding included (9 B)."""
    return 12 * valid + 9 * slots


def tis_weights(fb, dev, with_cpu=True):
    import torch

    from synthetic import ROLLOUT_TRAIN_BATCH, rollout_batch

    rb = rollout_batch(ROLLOUT_TRAIN_BATCH["responses"], ROLLOUT_TRAIN_BATCH["max_len"], (31, 1))
    lt, lr, adv = (torch.from_numpy(rb[k]).to(dev) for k in ("logp_train", "logp_rollout", "advantages"))
    msk = torch.from_numpy(rb["mask"]).to(dev)
    slots, valid = lt.numel(), int(rb["mask"].sum())
    byt = importance_weight_bytes(slots, valid)
    sets = [(t.clone() for t in (lt, lr, msk, adv)) for _ in range(rotations(21 * slots))]
    sets = [tuple(g) + (torch.empty_like(lt), torch.empty_like(lt)) for g in sets]
    ms, _ = _time_graph_ms([lambda t=t: fb.token_importance_weights(t[0], t[1], C=2.0, mode="tis", mask=t[2],
                                                                    advantages=t[3], out=t[4], out_adv=t[5])
                            for t in sets])
    gbps = byt / ms / 1e6
    res = {"tokens": valid, "slots": slots, "bytes": byt, "us": round(ms * 1e3, 1), "GBps": round(gbps, 1),
           "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
    if with_cpu:
        w, wa = fb.token_importance_weights(lt, lr, C=2.0, mode="tis", mask=msk, advantages=adv)
        res["cpu_baseline"], res["parity"] = tis_cpu_and_parity(rb, w.cpu().numpy(), wa.cpu().numpy(), byt)
    return res


# ---------------------------------------------------------------------------
# CPU oracle: parity of the timed runs and the CPU baseline, on the host's
# cores.  The oracle runs as it stands; the thread pool only splits it over
# independent pieces (128-row blocks of a weight, row chunks of activations),
# and its GEMM uses numpy's BLAS threads.
# ---------------------------------------------------------------------------

def _bits(t):
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pool_map(fn, items, threads):
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def _row_chunks(rows, step):
    return [(r, min(rows, r + step)) for r in range(0, rows, step)]


def oracle_quant_weight(w_bits, threads):
    """oracle.quant_weight_blockwise of [N][K] BF16 bits, one 128-row block
    row per task (blocks are independent)."""
    from oracle import quant_weight_blockwise

    res = _pool_map(lambda c: quant_weight_blockwise(w_bits[c[0]:c[1]]), _row_chunks(w_bits.shape[0], 128), threads)
    return np.concatenate([q for q, _ in res]), np.concatenate([s for _, s in res])


def oracle_quant_act(x_bits, threads):
    """oracle.quant_act_per_token_group in row chunks (tokens are independent)."""
    from oracle import quant_act_per_token_group

    res = _pool_map(lambda c: quant_act_per_token_group(x_bits[c[0]:c[1]]), _row_chunks(x_bits.shape[0], 16), threads)
    return np.concatenate([q for q, _ in res]), np.concatenate([s for _, s in res])


def _r14(y_bits, y_ref):
    """The 1e-2 acceptance of a GEMM output (relative Frobenius and worst
    element against max(|ref|, rms(ref))), with the BF16-exact fraction."""
    import oracle

    yf = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.asarray(y_ref, np.float64)
    rel_fro = float(np.linalg.norm(yf - ref) / np.linalg.norm(ref))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rel_max = float(np.max(np.abs(yf - ref) / np.maximum(np.abs(ref), rms)))
    exact = float(np.mean(y_bits == oracle.round_to_bf16_bits(ref)))
    return {"rel_fro": round(rel_fro, 6), "rel_max": round(rel_max, 6), "exact_bf16_frac": round(exact, 4),
            "pass": rel_fro <= 1e-2 and rel_max <= 1e-2}


def cpu_baseline_and_parity(fb, layers, w_bf16, sweep, gemm_flops):
    """Parity of the timed prefill step and of the re-quant sweep against the
    oracle, and the oracle's time for the same work on the host's cores.
    Codes are compared bit for bit with the GPU's fragment-order codes after
    the oracle's permutation, scales bit for bit.

    Prefill (the headline): per projection, 192 consecutive token rows (12
    groups of 16, at a seeded offset) are quantized by the oracle and
    multiplied by the FP32-accumulated oracle GEMM with the oracle's own
    weight codes (the whole matrix quantized by the oracle).  The GPU rows meet R14
    against it.  The oracle GEMM is timed at 64 and 192 rows; its time for
    all 8192 rows is the linear fit (a fixed part that decodes the weights,
    a per-row part), plus the per-row time of its activation quantizer.

    Re-quant sweep: the oracle quantizes the last layer's four matrices
    (batch index 35, byte offsets past 2^31 in the batched call) and layer 0
    in full, bit for bit against the GPU; its rate on those 386 M
    parameters gives the CPU time of the 36-layer sweep.
    """
    import torch

    from oracle import act_fragment_order, gemm_ref_fp32, quant_act_per_token_group

    threads = host_threads()
    M = PREFILL_M
    rng = np.random.default_rng(2024)
    r0 = int(rng.integers(0, (M - 192) // 16)) * 16
    par = {"prefill_qwen3_8b_layer": {"rows": [r0, r0 + 192], "weights_bitexact": True, "act_quant_bitexact": True,
                                      "gemm": {}}}
    pp = par["prefill_qwen3_8b_layer"]
    t_aq = t_fix = t_row = 0.0
    for L in layers:
        n, k = L["n"], L["k"]
        gq, gs = L["wq"].cpu().numpy(), L["ws"].cpu().numpy()
        qw, sw = oracle_quant_weight(_bits(w_bf16[L["name"]]), threads)
        pp["weights_bitexact"] &= bool(np.array_equal(gq, act_fragment_order(qw))
                                       and np.array_equal(gs.view(np.uint32), sw.view(np.uint32)))
        xb = _bits(L["x"][r0:r0 + 192])
        t = time.perf_counter()
        qa, sa = quant_act_per_token_group(xb)
        t_aq += (time.perf_counter() - t) / 192 * M
        frag = L["xq"].view(-1)[r0 * k:(r0 + 192) * k].cpu().numpy().reshape(192, k)
        pp["act_quant_bitexact"] &= bool(np.array_equal(frag, act_fragment_order(qa)) and np.array_equal(
            L["xs"][r0:r0 + 192].cpu().numpy().view(np.uint32), sa.view(np.uint32)))
        t = time.perf_counter()
        gemm_ref_fp32(qa[:64], sa[:64], qw, sw)
        t64 = time.perf_counter() - t
        t = time.perf_counter()
        ref = gemm_ref_fp32(qa, sa, qw, sw)
        t192 = time.perf_counter() - t
        per_row = max(0.0, (t192 - t64) / 128)
        t_row += per_row * M
        t_fix += max(0.0, t192 - 192 * per_row)
        pp["gemm"][L["name"]] = _r14(_bits(L["y"][r0:r0 + 192]), ref)
    pp["pass"] = pp["weights_bitexact"] and pp["act_quant_bitexact"] and all(g["pass"] for g in pp["gemm"].values())
    prefill_s = t_aq + t_fix + t_row

    # re-quant sweep: layers 35 and 0 of every projection, in full
    ps = {"layers_checked": [SWEEP_LAYERS - 1, 0], "bitexact": True}
    t_rq, params = 0.0, 0
    for name, w, q, s in sweep["tensors"]:
        for layer in (SWEEP_LAYERS - 1, 0):
            wb = _bits(w[layer])
            t = time.perf_counter()
            oq, os_ = oracle_quant_weight(wb, threads)
            t_rq += time.perf_counter() - t
            params += wb.size
            want = act_fragment_order(oq) if sweep["frag"] else oq
            ps["bitexact"] &= bool(np.array_equal(q[layer].cpu().numpy(), want) and np.array_equal(
                s[layer].cpu().numpy().view(np.uint32), os_.view(np.uint32)))
    ps["pass"] = ps["bitexact"]
    par["requant_sweep_36_layers"] = ps
    sweep_s = t_rq * sweep["params"] / params
    import threadpoolctl

    blas = [i.get("num_threads") for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    base = {
        "value": round(gemm_flops / prefill_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("prefill layer step: per projection 192 of the 8192 token rows (oracle act quant of those rows, "
                   "its FP32-accumulated GEMM timed at 64 and 192 rows), extrapolated to 8192 rows by a linear fit; "
                   "weights quantized beforehand as on the GPU; same input bytes as the GPU run"),
        "legs": {
            "prefill_layer_step": {"seconds_extrapolated": round(prefill_s, 3),
                                   "act_quant_s": round(t_aq, 3), "gemm_fixed_s": round(t_fix, 3),
                                   "gemm_rows_s": round(t_row, 3),
                                   "TFLOPs": round(gemm_flops / prefill_s / 1e12, 6),
                                   "threads": {"act_quant": 1, "gemm_blas": blas[0] if blas else None}},
            "requant_sweep_36_layers": {"sample": "layers 35 and 0 of the four projections (386 M params), "
                                                  "extrapolated to 6.95 G", "seconds_sample": round(t_rq, 3),
                                        "seconds_extrapolated": round(sweep_s, 3),
                                        "GBps": round(sweep["bytes"] / sweep_s / 1e9, 3),
                                        "threads": threads},
        },
        "host": {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                 "blas": [i.get("internal_api") for i in threadpoolctl.threadpool_info()
                          if i.get("user_api") == "blas"]},
    }
    par["pass"] = pp["pass"] and ps["pass"]
    return base, par


def train_cpu_and_parity(checks):
    """The oracle's dual quantizers on the same input bytes: W and W^T of the
    last and first layer of every projection from the 36-layer batch calls,
    and both activations' x and x^T, all compared bit for bit (codes and
    scale bits).  Its time per byte of algorithmic traffic is the baseline."""
    from oracle.train import quant_act_dual

    threads = host_threads()
    ok, t_w, t_x, b_w, b_x = {}, 0.0, 0.0, 0, 0
    for label, xb, gpu in checks:
        t0 = time.perf_counter()
        if label.startswith("W"):  # quant_weight_blockwise_dual: W and W^T, block rows on the thread pool
            ref = oracle_quant_weight(xb, threads) + oracle_quant_weight(np.ascontiguousarray(xb.T), threads)
            t_w += time.perf_counter() - t0
            b_w += xb.size * 4 + sum(r.size * 4 for r in ref[1::2])
        else:
            ref = sum(quant_act_dual(xb), ())
            t_x += time.perf_counter() - t0
            b_x += xb.size * 4 + sum(r.size * 4 for r in ref[1::2])
        ok[label] = bool(all(np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                                            r.view(np.uint32) if r.dtype == np.float32 else r)
                             for g, r in zip(gpu, ref)))
    base = {"kind": "oracle", "threads": threads, "unit": "GB/s",
            "sample": "layers 35 and 0 of each projection (W and W^T), both activations (x and x^T)",
            "weight_dual_GBps": round(b_w / t_w / 1e9, 3) if t_w else None,
            "act_dual_GBps": round(b_x / t_x / 1e9, 3) if t_x else None,
            "seconds": {"weights": round(t_w, 3), "activations": round(t_x, 3)}}
    return base, {"bitexact": ok, "pass": all(ok.values())}


def kv_cpu_and_parity(bits, ks, vs, kc, vc, cal_bytes, wr_bytes):
    """The oracle's per-head K and V calibration over all 16,384 tokens
    (scales bit for bit), the prefill write of those tokens into slots
    0..T-1 and the decode write of 1,536 more tokens after them (every
    cache byte compared, with the oracle's own scales)."""
    from oracle.kv import kv_calibrate, kv_quantize

    k, v, kn, vn = bits
    T = k.shape[0]
    t0 = time.perf_counter()
    rks, rvs = kv_calibrate(k, True), kv_calibrate(v, True)
    t_cal = time.perf_counter() - t0
    t0 = time.perf_counter()
    rkc, rvc = kv_quantize(k, rks, True), kv_quantize(v, rvs, True)
    t_wr = time.perf_counter() - t0
    rkd, rvd = kv_quantize(kn, rks, True), kv_quantize(vn, rvs, True)
    par = {"scales_bitexact": bool(np.array_equal(ks.view(np.uint32), rks.view(np.uint32))
                                   and np.array_equal(vs.view(np.uint32), rvs.view(np.uint32))),
           "prefill_write_bitexact": bool(np.array_equal(kc[:T], rkc) and np.array_equal(vc[:T], rvc)),
           "decode_write_bitexact": bool(np.array_equal(kc[T:], rkd) and np.array_equal(vc[T:], rvd))}
    par["pass"] = all(par.values())
    base = {"kind": "oracle", "threads": 1, "unit": "GB/s", "sample": "the whole calibration and prefill write",
            "calibrate_GBps": round(cal_bytes / t_cal / 1e9, 3), "write_GBps": round(wr_bytes / t_wr / 1e9, 3),
            "seconds": {"calibrate": round(t_cal, 3), "write": round(t_wr, 3)}}
    return base, par


def tis_cpu_and_parity(rb, w, wa, byt):
    """The oracle's TIS weights of the whole batch: every slot's w within
    2 ulp and w * A within 6 ulp of the oracle's correctly rounded values,
    NaN, zero and infinity positions identical (the GPU tests' bar)."""
    from oracle.tis import TIS, importance_weights

    t0 = time.perf_counter()
    rw, rwa = importance_weights(rb["logp_train"], rb["logp_rollout"], C=2.0, mode=TIS, mask=rb["mask"],
                                 advantages=rb["advantages"])
    t = time.perf_counter() - t0

    def ulps(g, r):
        g, r = np.asarray(g, np.float32), np.asarray(r, np.float32)
        same_special = bool(np.array_equal(np.isnan(g), np.isnan(r)) and np.array_equal(g == 0, r == 0)
                            and np.array_equal(g[np.isinf(r)], r[np.isinf(r)]))
        fin = np.isfinite(r) & ~np.isnan(r)
        err = np.abs(g[fin].astype(np.float64) - r[fin]) / np.maximum(
            np.spacing(np.abs(r[fin])).astype(np.float64), 2.0 ** -149)
        return same_special, float(err.max()) if err.size else 0.0

    sw, ew = ulps(w, rw)
    sa, ea = ulps(wa, rwa)
    par = {"w_max_ulp": round(ew, 3), "wA_max_ulp": round(ea, 3), "special_values_equal": sw and sa}
    par["pass"] = bool(sw and sa and ew <= 2.0 and ea <= 6.0)
    base = {"kind": "oracle", "threads": 1, "unit": "GB/s", "sample": "the whole batch",
            "value": round(byt / t / 1e9, 3), "seconds": round(t, 3)}
    return base, par


MOE_PARITY_TOKENS = 16
MOE_TIMING_EXPERTS = 2


def moe_cpu_and_parity(x, ids, tw, w1, w2, w1q, w1s, w2q, w2s, off, sp, pr, out, hq, y2, layer_flops, req_bytes):
    """The oracle on the MoE layer's input bytes.

    Parity (as in the GPU tests' layer check): the routing sort of all pairs
    (bit for bit); the weights of every expert used below, re-quantized by
    the oracle (bit for bit against the GPU's codes and scales);
    MOE_PARITY_TOKENS sampled tokens' whole chain (act quant, fc1,
    SiLU(gate) * up and its 1x128 quantization, fc2, weighted combine)
    against the GPU layer output: 1e-2 in Frobenius norm and
    min(2^-4, 1/sqrt(F)) per element.  For all rows of MOE_TIMING_EXPERTS
    sampled experts: the h codes (equal to the oracle's for >= 99% of them:
    where the GPU's and the oracle's fc1 outputs, each within the GEMM bar,
    round to BF16 differently, a code can sit one E4M3 step apart) and the
    fc2 outputs in Frobenius norm (1e-2; a flipped code of a large h moves a
    single fc2 row by more than the per-element bar, which holds for the
    routing-weighted sum of a token's rows).

    CPU baseline: the oracle's time for the sort, the act quant of all
    tokens, the fc1 -> SiLU * up quant -> fc2 chain of all rows of the
    sampled experts (scaled to all experts) and the combine of all pairs
    (on host-drawn BF16 rows of the same shape); expert re-quant per
    parameter, scaled to all experts."""
    from oracle import dequant_act, dequant_weight, round_to_bf16_bits
    from oracle.bf16 import bf16_bits_to_f64
    from oracle.moe import combine, silu_mul_quantize, sort_by_expert

    threads = host_threads()
    T, H = x.shape
    E, F, k = w1.shape[0], w2.shape[2], ids.shape[1]
    bar = float(min(2.0 ** -4, 1.0 / np.sqrt(F)))

    def layer_bar(y_bits, ref):
        rep = _r14(y_bits, ref)
        rep["pass"] = bool(rep["rel_fro"] <= 1e-2 and rep["rel_max"] <= bar)
        rep["rel_max_bar"] = round(bar, 6)
        return rep

    t0 = time.perf_counter()
    roff, rrows, rpr = sort_by_expert(ids, E)
    t_sort = time.perf_counter() - t0
    off_h, sp_h, pr_h = off.cpu().numpy(), sp.cpu().numpy(), pr.cpu().numpy()
    sort_ok = bool(np.array_equal(off_h, roff) and np.array_equal(sp_h[:roff[-1]], rrows)
                   and np.array_equal(pr_h, rpr))

    rng = np.random.default_rng([70, 1])
    toks = np.sort(rng.choice(T, size=MOE_PARITY_TOKENS, replace=False))
    busy = np.nonzero(np.diff(roff) > 0)[0]  # experts with routed rows
    texp = np.sort(rng.choice(busy, size=min(MOE_TIMING_EXPERTS, busy.size), replace=False))
    used = np.union1d(np.unique(ids[toks]), texp).astype(int)
    t0 = time.perf_counter()
    wo = {int(e): (oracle_quant_weight(_bits(w1[int(e)]), threads), oracle_quant_weight(_bits(w2[int(e)]), threads))
          for e in used}
    t_rq = time.perf_counter() - t0
    req_ok = True
    for e, pair in wo.items():
        for (q, sc), gq, gs in zip(pair, (w1q[e], w2q[e]), (w1s[e], w2s[e])):
            req_ok &= bool(np.array_equal(gq.cpu().numpy(), q)
                           and np.array_equal(gs.cpu().numpy().view(np.uint32), sc.view(np.uint32)))

    xb = _bits(x)
    t0 = time.perf_counter()
    aq, asc = oracle_quant_act(xb, threads)
    t_aq = time.perf_counter() - t0

    wd = {}

    def fc_chain(e, rows_q, rows_s):
        if e not in wd:
            wd[e] = (dequant_weight(*wo[e][0]), dequant_weight(*wo[e][1]))
        y1 = dequant_act(rows_q, rows_s) @ wd[e][0].T
        h_q, h_s = silu_mul_quantize(round_to_bf16_bits(y1), F)
        return h_q, round_to_bf16_bits(dequant_act(h_q, h_s) @ wd[e][1].T)

    # the sampled experts: all their rows, timed
    t0 = time.perf_counter()
    ref_e = {}
    for e in texp:
        e = int(e)
        tok = rrows[roff[e]:roff[e + 1]] // k
        ref_e[e] = fc_chain(e, aq[tok], asc[tok])
    t_ex = time.perf_counter() - t0
    hq_h, y2_h = hq.cpu().numpy(), _bits(y2)
    experts_rep = {}
    for e, (h_ref, y_ref) in ref_e.items():
        rep = _r14(y2_h[roff[e]:roff[e + 1]], bf16_bits_to_f64(y_ref))
        same = float(np.mean(hq_h[roff[e]:roff[e + 1]] == h_ref))
        rep.update({"h_codes_equal_frac": round(same, 5), "pass": bool(rep["rel_fro"] <= 1e-2 and same >= 0.99)})
        experts_rep[str(e)] = rep

    # the sampled tokens' whole chain against the layer output
    ref = np.zeros((toks.size, H))
    for j in range(k):
        for t_i, t in enumerate(toks):
            e = int(ids[t, j])
            ref[t_i] += float(tw[t, j]) * bf16_bits_to_f64(fc_chain(e, aq[t:t + 1], asc[t:t + 1])[1][0])
    layer_rep = layer_bar(_bits(out)[toks], ref)

    # the combine of all pairs, on host-drawn BF16 rows (timing only)
    yc = round_to_bf16_bits(np.random.default_rng([70, 2]).standard_normal((T * k, H)))
    t0 = time.perf_counter()
    combine(yc, rpr, tw)
    t_comb = time.perf_counter() - t0

    params_used = int(used.size) * (w1[0].numel() + w2[0].numel())
    t_req_all = t_rq * (w1.numel() + w2.numel()) / params_used
    t_layer = t_sort + t_aq + t_ex * E / texp.size + t_comb
    base = {"value": round(layer_flops / t_layer / 1e12, 6), "unit": "TFLOP/s", "threads": threads,
            "kind": "oracle",
            "sample": ("MoE layer: sort of all %d pairs, act quant of all %d tokens, the fc1 -> SiLU*up quant -> "
                       "fc2 chain of all rows of %d experts scaled to %d experts, combine of all pairs; expert "
                       "re-quant of %d experts scaled to all %d by parameters"
                       % (T * k, T, texp.size, E, used.size, E)),
            "expert_requant_GBps": round(req_bytes / t_req_all / 1e9, 3),
            "seconds": {"sort": round(t_sort, 3), "act_quant": round(t_aq, 3),
                        "experts_sampled": round(t_ex, 3), "combine": round(t_comb, 3),
                        "layer_extrapolated": round(t_layer, 3), "requant_sampled": round(t_rq, 3),
                        "expert_requant_extrapolated": round(t_req_all, 3)}}
    par = {"tokens": toks.tolist(), "experts": [int(e) for e in texp], "experts_requant_checked": int(used.size),
           "sort_bitexact": sort_ok, "expert_requant_bitexact": req_ok, "fc2_rows_of_experts": experts_rep,
           "layer_tokens": layer_rep}
    par["pass"] = bool(sort_ok and req_ok and layer_rep["pass"] and all(r["pass"] for r in experts_rep.values()))
    return base, par


def torch_index(idx, device):
    import torch

    return torch.from_numpy(np.asarray(idx, np.int64)).to(device)


def decode_cpu_and_parity(layers, m, flops):
    """The oracle runs the whole decode step on the same input bytes: weight
    re-quant (thread pool over block rows), act quant, FP32-accumulated GEMM
    (BLAS threads); its outputs check the GPU's bit for bit (quantizers) and
    by R14 (GEMMs)."""
    from oracle import act_fragment_order, gemm_ref_fp32, quant_act_per_token_group

    threads = host_threads()
    host = [(_bits(L["w"]), _bits(L["x"])) for L in layers]
    t0 = time.perf_counter()
    wres = [oracle_quant_weight(w, threads) for w, _ in host]
    t_rq = time.perf_counter() - t0
    t0 = time.perf_counter()
    ares = [quant_act_per_token_group(x) for _, x in host]
    t_aq = time.perf_counter() - t0
    t0 = time.perf_counter()
    yres = [gemm_ref_fp32(qa, sa, qw, sw) for (qa, sa), (qw, sw) in zip(ares, wres)]
    t_gm = time.perf_counter() - t0
    total = t_rq + t_aq + t_gm
    base = {"value": round(flops / total / 1e12, 6), "unit": "TFLOP/s", "threads": threads, "kind": "oracle",
            "sample": "the whole decode layer step, same input bytes",
            "seconds": {"requant": round(t_rq, 3), "act_quant": round(t_aq, 3), "gemm": round(t_gm, 3)}}
    par = {"requant_bitexact": True, "act_quant_bitexact": True, "gemm": {}}
    for L, (qw, sw), (qa, sa), y_ref in zip(layers, wres, ares, yres):
        par["requant_bitexact"] &= bool(np.array_equal(L["wq"].cpu().numpy(), act_fragment_order(qw))
                                        and np.array_equal(L["ws"].cpu().numpy().view(np.uint32),
                                                           sw.view(np.uint32)))
        par["act_quant_bitexact"] &= bool(np.array_equal(L["xq"].cpu().numpy(), act_fragment_order(qa))
                                          and np.array_equal(L["xs"].cpu().numpy().view(np.uint32),
                                                             sa.view(np.uint32)))
        par["gemm"][L["name"]] = _r14(_bits(L["y"]), y_ref)
    par["pass"] = par["requant_bitexact"] and par["act_quant_bitexact"] and all(g["pass"] for g in par["gemm"].values())
    return base, par


# ---------------------------------------------------------------------------
# rocprofv3 summary of this benchmark (kernel trace + HBM byte counters)
# ---------------------------------------------------------------------------

def _csv_rows(pattern):
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(kernel_name):
    """Kernel name without the namespace prefix and the parameter list."""
    n = re.sub(r"^void ", "", kernel_name)
    n = n.replace("fp8bq::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):  # cut at the '(' of the parameter list (outside template brackets)
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return n[:i]
    return n


def _phase_of(kernel_name):
    for p, (prefix, _) in PHASE_KERNELS.items():
        if prefix in kernel_name and not (p == "requant" and "quant_weight_multi" in kernel_name):
            return p
    return None


def step_algorithmic_bytes():
    """Average algorithmic HBM bytes per launch of each measured phase."""
    sys.path.insert(0, ROOT)
    from synthetic import LAYER_SHAPES_QWEN3_8B

    M = PREFILL_M
    aq = gm = rq = 0
    for _, n, k in LAYER_SHAPES_QWEN3_8B:
        ws = (n // 128) * (k // 128) * 4
        xs = M * (k // 128) * 4
        aq += M * k * 3 + xs
        gm += M * k + n * k + 2 * M * n + xs + ws
        rq += SWEEP_LAYERS * (n * k * 3 + ws)
    return {"act_quant": aq / PHASE_LAUNCHES["act_quant"], "gemm": gm / PHASE_LAUNCHES["gemm"],
            "requant": rq / PHASE_LAUNCHES["requant"]}


def _copy_scale(d, sub, counter):
    v = [float(r["Counter_Value"]) * 1024.0 for r in _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv"))
         if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    return float(1 << 30) / (sum(v) / len(v)) if v else None


def rocprof_summary(d):
    """Markdown summary of the rocprofv3 runs under `d`:
      d/kt/**/*kernel_stats.csv           --kernel-trace --stats of this benchmark
      d/fetch/**/*counter_collection.csv  --pmc FETCH_SIZE of this benchmark
      d/write/**/*counter_collection.csv  --pmc WRITE_SIZE of this benchmark
      d/copy_fetch, d/copy_write          the same counters for --calibrate-copy
    Counter values are KiB per dispatch; each is scaled by (bytes the copy
    really moves) / (what the counter reads for the copy)."""
    lines = []
    stats = _csv_rows(os.path.join(d, "kt", "**", "*kernel_stats.csv"))
    lines.append("| kernel | calls | avg duration (us) | total (ms) |")
    lines.append("|---|---|---|---|")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        short = _short(r["Name"])
        lines.append("| `%s` | %s | %.2f | %.3f |" % (short[:110], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                      float(r["TotalDurationNs"]) / 1e6))

    def per_dispatch(sub, counter):
        vals = {}
        for r in _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    scale = {"FETCH_SIZE": _copy_scale(d, "copy_fetch", "FETCH_SIZE"),
             "WRITE_SIZE": _copy_scale(d, "copy_write", "WRITE_SIZE")}
    lines.append("")
    lines.append("Copy calibration (1 GiB read + 1 GiB written per launch): FETCH_SIZE scale %s, "
                 "WRITE_SIZE scale %s." % tuple("%.3f" % scale[c] if scale[c] else "n/a"
                                                  for c in ("FETCH_SIZE", "WRITE_SIZE")))
    lines.append("")
    lines.append("| kernel | dispatches | HBM read / launch (MB) | HBM write / launch (MB) |")
    lines.append("|---|---|---|---|")
    fetch = per_dispatch("fetch", "FETCH_SIZE")
    write = per_dispatch("write", "WRITE_SIZE")
    traffic = {}
    for name in sorted(set(fetch) | set(write)):
        p = _phase_of(name)
        f = fetch.get(name, [])
        w = write.get(name, [])
        fr = sum(f) / len(f) * (scale["FETCH_SIZE"] or float("nan")) if f else float("nan")
        wr = sum(w) / len(w) * (scale["WRITE_SIZE"] or float("nan")) if w else float("nan")
        lines.append("| `%s` | %d | %.2f | %.2f |" % (_short(name)[:110], max(len(f), len(w)),
                                                      fr / 1e6, wr / 1e6))
        if p and f and w:
            t = traffic.setdefault(p, {"n": 0, "bytes": 0.0})
            t["n"] += 1
            t["bytes"] += fr + wr
    out = {p: {"bytes_per_launch": int(t["bytes"] / t["n"]), "source_sha": source_sha(PHASE_KERNELS[p][1])}
           for p, t in traffic.items()}
    algo = step_algorithmic_bytes()
    lines.append("")
    lines.append("| phase | measured HBM bytes / launch (MB) | algorithmic bytes / launch (MB) | ratio |")
    lines.append("|---|---|---|---|")
    for p, v in sorted(out.items()):
        a = algo[p]
        lines.append("| %s | %.2f | %.2f | %.3f |" % (p, v["bytes_per_launch"] / 1e6, a / 1e6, v["bytes_per_launch"] / a))
    lines.append("")
    lines.append("traffic-json: " + json.dumps(out, sort_keys=True))
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# GEMM counter profile: each GEMM of the decode (M = 256), prefill (M = 8192)
# and MoE expert configurations, GEMM_PROFILE_REPS launches in a row, in
# this order; the summary matches GEMM dispatches to cases by that order.
# ---------------------------------------------------------------------------

GEMM_PROFILE_REPS = 3


def gemm_profile_cases():
    """(label, M_total, N, K, experts or 0) of every GEMM profiled, in launch order."""
    sys.path.insert(0, ROOT)
    from synthetic import LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B

    # decode and "prefill frag": both operands in fragment order (the
    # library's path at these shapes); "prefill": both row-major
    cases = [("decode %s" % nm, 256, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    cases += [("prefill %s" % nm, 8192, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    cases += [("prefill frag %s" % nm, 8192, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    moe = MOE_QWEN3_30B_A3B
    mt = moe["tokens"] * moe["top_k"]
    cases.append(("MoE fc1 gate_up", mt, moe["gate_up"][0], moe["gate_up"][1], moe["experts"]))
    cases.append(("MoE fc2 down", mt, moe["down"][0], moe["down"][1], moe["experts"]))
    # fc1 with SiLU(gate) * up quantized in its epilogue: N = 2F columns
    # computed, F codes + F/128 scales per row stored
    cases.append(("MoE fc1 gate_up + SiLU quant (fused)", mt, moe["gate_up"][0], moe["gate_up"][1], moe["experts"]))
    return cases


def gemm_profile():
    """Run each case GEMM_PROFILE_REPS times on freshly quantized synthetic inputs."""
    import torch

    sys.path.insert(0, ROOT)
    import fp8_blockwise_quantized_quantize_amd as fb
    from synthetic import MOE_QWEN3_30B_A3B, device_bf16_normal, moe_routing

    moe = MOE_QWEN3_30B_A3B
    _, _, off = moe_routing(moe["tokens"], moe["experts"], moe["top_k"], (4, 0))
    offsets = torch.from_numpy(off).to("cuda:0")
    for i, (label, m, n, k, g) in enumerate(gemm_profile_cases()):
        w = device_bf16_normal((g, n, k) if g else (n, k), 0.02, seed=700 + i)
        x = device_bf16_normal((m, k), 1.0, seed=800 + i)
        frag = label.startswith("decode") or label.startswith("prefill frag")
        if frag:
            wq, ws = fb.quantize_weight_blockwise_frag(w)
            xq, xs = fb.quantize_act_per_token_group_frag(x)
        else:
            wq, ws = fb.quantize_weight_blockwise(w)
            xq, xs = fb.quantize_act_per_token_group(x)
        del w, x
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        fused = "fused" in label
        if fused:
            rows = torch.arange(m, dtype=torch.int32, device="cuda:0")
            h = torch.empty((m, n // 2), dtype=torch.uint8, device="cuda:0")
            hs = torch.empty((m, n // 2 // 128), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        for _ in range(GEMM_PROFILE_REPS):
            if frag:
                fb.gemm_w8a8_blockscaled_frag(xq, xs, wq, ws, y)
            elif fused:
                fb.grouped_gemm_w8a8_blockscaled_gather_silu(xq, xs, rows, 1, wq, ws, offsets, h, hs)
            elif g:
                fb.grouped_gemm_w8a8_blockscaled(xq, xs, wq, ws, offsets, y)
            else:
                fb.gemm_w8a8_blockscaled(xq, xs, wq, ws, y)
        torch.cuda.synchronize()
        print("gemm profile case done:", label, flush=True)
        del wq, ws, xq, xs, y
        torch.cuda.empty_cache()


def gemm_counter_summary(d):
    """Markdown summary of the rocprofv3 passes of --gemm-profile under `d`:
      kt     --kernel-trace            durations per dispatch
      mfma   SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE
      lds    SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_LDS_ADDR_CONFLICT
      l2     TCC_HIT_sum TCC_MISS_sum
      wave   SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS
             SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_ANY
      ta     TA_BUSY_avr GRBM_GUI_ACTIVE
      fetch / write, copy_fetch / copy_write   as for the benchmark summary
    MOPS_F8 counts FP8 MFMA work in units of 512 FLOPs (it equals 2MNK on
    dense shapes).  GRBM_GUI_ACTIVE reads 8 x the kernel's cycles (it sums
    over the 8 XCDs: / 8 / duration gives 2.0-2.2 GHz on the long prefill
    kernels), so the clock is GRBM_GUI_ACTIVE / 8 / duration (meaningful for
    long kernels only: the counter window also covers launch overhead).
    MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); it equals
    the FLOP rate over the FP8 peak at the measured clock."""
    cases = gemm_profile_cases()

    def gemm_dispatches(rows, key):
        out = {}
        for r in rows:
            if "gemm_dense_kernel" in r["Kernel_Name"] or "gemm_grouped" in r["Kernel_Name"]:
                out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]}).update(key(r))
        return [out[i] for i in sorted(out)]

    def counters(sub):
        rows = _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv"))
        return gemm_dispatches(rows, lambda r: {r["Counter_Name"]: float(r["Counter_Value"])})

    kt = gemm_dispatches(_csv_rows(os.path.join(d, "kt", "**", "*kernel_trace.csv")),
                         lambda r: {"ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
    passes = {sub: counters(sub) for sub in ("mfma", "lds", "l2", "fetch", "write", "wave", "ta")}
    n_expected = len(cases) * GEMM_PROFILE_REPS

    def per_case(disp, key):
        if len(disp) != n_expected:
            return [None] * len(cases)
        vals = []
        for c in range(len(cases)):
            xs = [x.get(key) for x in disp[c * GEMM_PROFILE_REPS:(c + 1) * GEMM_PROFILE_REPS]]
            xs = [x for x in xs if x is not None]
            vals.append(sum(xs) / len(xs) if xs else None)
        return vals

    copy = {"FETCH_SIZE": _copy_scale(d, "copy_fetch", "FETCH_SIZE"),
            "WRITE_SIZE": _copy_scale(d, "copy_write", "WRITE_SIZE")}
    ns = per_case(kt, "ns")
    mops = per_case(passes["mfma"], "SQ_INSTS_VALU_MFMA_MOPS_F8")
    busy = per_case(passes["mfma"], "SQ_VALU_MFMA_BUSY_CYCLES")
    grbm = per_case(passes["mfma"], "GRBM_GUI_ACTIVE")
    bank = per_case(passes["lds"], "SQ_LDS_BANK_CONFLICT")
    ldsact = per_case(passes["lds"], "SQ_LDS_IDX_ACTIVE")
    hit = per_case(passes["l2"], "TCC_HIT_sum")
    miss = per_case(passes["l2"], "TCC_MISS_sum")
    fetch = per_case(passes["fetch"], "FETCH_SIZE")
    write = per_case(passes["write"], "WRITE_SIZE")
    names = [_short(kt[c * GEMM_PROFILE_REPS]["name"]) if len(kt) == n_expected else "?" for c in range(len(cases))]

    def f(v, fmt):
        return fmt % v if v is not None else "n/a"

    lines = ["Dispatches matched: kernel trace %d, mfma %d, lds %d, l2 %d, fetch %d, write %d (expected %d)."
             % (len(kt), *(len(passes[s]) for s in ("mfma", "lds", "l2", "fetch", "write")), n_expected), "",
             "| GEMM | kernel | us | TFLOP/s (2MNK) | % of FP8 peak | counter FLOPs / 2MNK | clock GHz "
             "| MFMA busy | LDS bank-conflict / active cycles | L2 hit | L2-miss MB / algorithmic MB |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for c, (label, m, n, k, g) in enumerate(cases):
        flops = 2.0 * m * n * k
        nb = -(-n // 128)
        out_b = m * (n // 2) + 4 * m * (n // 256) + 4 * m if "fused" in label else 2 * m * n  # + gather index
        algo = m * k + (g or 1) * n * k + out_b + 4 * m * (k // 128) + 4 * (g or 1) * nb * (k // 128)
        tf = flops / ns[c] / 1e3 if ns[c] else None
        ghz = grbm[c] / 8.0 / ns[c] if grbm[c] and ns[c] else None
        mb = busy[c] / (grbm[c] / 8.0 * 1024.0) if busy[c] is not None and grbm[c] else None
        hbm = None
        if fetch[c] is not None and write[c] is not None and copy["FETCH_SIZE"] and copy["WRITE_SIZE"]:
            hbm = (fetch[c] * 1024.0 * copy["FETCH_SIZE"] + write[c] * 1024.0 * copy["WRITE_SIZE"]) / 1e6
        lines.append("| %s (M=%d N=%d K=%d%s) | `%s` | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            label, m, n, k, ", %d experts" % g if g else "", names[c][:60], f(ns[c] and ns[c] / 1e3, "%.1f"),
            f(tf, "%.0f"), f(tf and 100.0 * tf / FP8_PEAK_TFLOPS, "%.1f%%"),
            f(mops[c] and mops[c] * 512.0 / flops, "%.3f"), f(ghz, "%.2f"), f(mb and 100.0 * mb, "%.1f%%"),
            f(bank[c] / ldsact[c] if bank[c] is not None and ldsact[c] else None, "%.3f"),
            f(hit[c] / (hit[c] + miss[c]) if hit[c] is not None and miss[c] is not None and hit[c] + miss[c] else None,
              "%.3f"),
            f(hbm and "%.1f / %.1f" % (hbm, algo / 1e6), "%s")))
    # where the waves' time goes: each counter over SQ_WAVE_CYCLES (wave-cycles
    # summed over waves); TA busy over the kernel's cycles (ta pass)
    wc = per_case(passes["wave"], "SQ_WAVE_CYCLES")
    wave_cols = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                 "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM")
    wv = {c: per_case(passes["wave"], c) for c in wave_cols}
    ta = per_case(passes["ta"], "TA_BUSY_avr")
    ta_grbm = per_case(passes["ta"], "GRBM_GUI_ACTIVE")
    lines += ["", "Dispatches matched: wave %d, ta %d (expected %d).  Fractions of the waves' cycles "
              "(SQ_WAVE_CYCLES), and TA busy over the kernel's cycles:" % (len(passes["wave"]), len(passes["ta"]),
                                                                          n_expected), "",
              "| GEMM | " + " | ".join(c.replace("SQ_", "") for c in wave_cols) + " | TA busy |",
              "|---" * (len(wave_cols) + 2) + "|"]
    for c, (label, m, n, k, g) in enumerate(cases):
        cells = [f(wv[col][c] / wc[c] if wv[col][c] is not None and wc[c] else None, "%.3f") for col in wave_cols]
        tb = ta[c] / (ta_grbm[c] / 8.0) if ta[c] is not None and ta_grbm[c] else None
        lines.append("| %s | %s | %s |" % (label, " | ".join(cells), f(tb, "%.3f")))
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# Bandwidth-bound kernels: each runs BW_PROFILE_REPS times on its
# configuration's shape, in the order of bw_profile_cases(); the summary
# matches dispatches to cases by that order and compares the HBM bytes the
# counters measure with the algorithmic bytes of each case.
# ---------------------------------------------------------------------------

BW_PROFILE_REPS = 3


def bw_profile_cases():
    """(label, kernel-name prefix, algorithmic bytes per launch) in launch order."""
    sys.path.insert(0, ROOT)
    from synthetic import LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B

    cases = []
    for nm, n, k in LAYER_SHAPES_QWEN3_8B:  # 36-layer sweep: one call per projection, fragment order
        cases.append(("requant sweep %s (batch 36)" % nm, "quant_weight_kernel",
                      SWEEP_LAYERS * (n * k * 3 + (n // 128) * (k // 128) * 4)))
    for k in (4096, 12288):
        ab = PREFILL_M * k * 3 + PREFILL_M * (k // 128) * 4
        cases.append(("prefill act quant 8192x%d" % k, "quant_act_kernel", ab))
        cases.append(("prefill act quant frag 8192x%d" % k, "quant_act_frag_kernel", ab))
    cases.append(("decode act quant frag, 4 activations (one launch)", "quant_act_frag_multi_kernel",
                  sum(256 * k * 3 + 256 * (k // 128) * 4 for _, _, k in LAYER_SHAPES_QWEN3_8B)))
    cases.append(("decode requant frag, 4 matrices (one launch)", "quant_weight_multi_kernel",
                  sum(n * k * 3 + (n // 128) * (k // 128) * 4 for _, n, k in LAYER_SHAPES_QWEN3_8B)))
    moe = MOE_QWEN3_30B_A3B
    T, k, H, F = moe["tokens"], moe["top_k"], moe["hidden"], moe["ffn"]
    R = T * k
    cases.append(("MoE token act quant 4096x2048", "quant_act_kernel", T * H * 3 + T * (H // 128) * 4))
    cases.append(("MoE SiLU*up quant 32768x768", "silu_mul_quant_kernel", R * 2 * F * 2 + R * F + R * (F // 128) * 4))
    cases.append(("MoE combine 4096x2048 (top-8)", "combine_kernel", R * H * 2 + R * 8 + T * H * 2))
    Tk, Hk, D = 16384, 8, 128
    cases.append(("KV calibrate 16384 tokens", "kv_amax_kernel", 2 * Tk * Hk * D * 2))
    cases.append(("KV write 16384 tokens", "kv_write_kernel", 2 * Tk * Hk * D * 3 + Tk * 4))
    cases.append(("TIS weights 512x20000", "importance_weight_kernel", None))
    cases.append(("W/W^T dual quant gate_up (batch 36)", "dual_quant_kernel",
                  SWEEP_LAYERS * (24576 * 4096 * 4 + 2 * (24576 // 128) * (4096 // 128) * 4)))
    cases.append(("x/x^T dual quant 8192x4096", "dual_quant_kernel",
                  PREFILL_M * 4096 * 4 + PREFILL_M * 32 * 4 + 4096 * (PREFILL_M // 128) * 4))
    return cases


def bw_profile():
    """Run each bandwidth-bound case BW_PROFILE_REPS times (freshly generated inputs)."""
    import torch

    sys.path.insert(0, ROOT)
    import fp8_blockwise_quantized_quantize_amd as fb
    from synthetic import (LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B, ROLLOUT_TRAIN_BATCH, device_bf16_normal,
                           moe_topk, rollout_batch)

    dev = torch.device("cuda:0")
    R = BW_PROFILE_REPS

    def done(label):
        torch.cuda.synchronize()
        print("bw profile case done:", label, flush=True)
        torch.cuda.empty_cache()

    for p, (nm, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((SWEEP_LAYERS, n, k), 0.02, seed=800 + p)
        q = torch.empty((SWEEP_LAYERS, n, k), dtype=torch.uint8, device=dev)
        s = torch.empty((SWEEP_LAYERS, n // 128, k // 128), dtype=torch.float32, device=dev)
        for _ in range(R):
            fb.quantize_weight_blockwise_frag(w, q, s)
        del w, q, s
        done("requant sweep " + nm)
    for k in (4096, 12288):
        x = device_bf16_normal((PREFILL_M, k), 1.0, seed=960 + k)
        q = torch.empty((PREFILL_M, k), dtype=torch.uint8, device=dev)
        s = torch.empty((PREFILL_M, k // 128), dtype=torch.float32, device=dev)
        for _ in range(R):
            fb.quantize_act_per_token_group(x, q, s)
        torch.cuda.synchronize()
        for _ in range(R):
            fb.quantize_act_per_token_group_frag(x, q, s)
        del x, q, s
        done("prefill act quant %d" % k)
    xs = [device_bf16_normal((256, k), 1.0, seed=200 + i) for i, (_, _, k) in enumerate(LAYER_SHAPES_QWEN3_8B)]
    for _ in range(R):
        fb.quantize_acts_per_token_group_frag_multi(xs)
    ws = [device_bf16_normal((n, k), 0.02, seed=100 + i) for i, (_, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B)]
    torch.cuda.synchronize()
    for _ in range(R):
        fb.quantize_weights_blockwise_frag_multi(ws)
    del xs, ws
    done("decode multi")
    moe = MOE_QWEN3_30B_A3B
    T, E, k, H, F = moe["tokens"], moe["experts"], moe["top_k"], moe["hidden"], moe["ffn"]
    x = device_bf16_normal((T, H), 1.0, seed=700)
    for _ in range(R):
        fb.quantize_act_per_token_group(x)
    y1 = device_bf16_normal((T * k, 2 * F), 1.0, seed=701)
    torch.cuda.synchronize()
    for _ in range(R):
        fb.silu_mul_quantize_act(y1)
    ids_h, tw_h = moe_topk(T, E, k, (70, 0))
    ids, tw = torch.from_numpy(ids_h).to(dev), torch.from_numpy(tw_h).to(dev)
    _, _, pr = fb.moe_sort_by_expert(ids, E)
    y2 = device_bf16_normal((T * k, H), 1.0, seed=702)
    torch.cuda.synchronize()
    for _ in range(R):
        fb.moe_combine(y2, pr, tw)
    del x, y1, y2
    done("moe glue")
    Tk, Hk, D = 16384, 8, 128
    kk = device_bf16_normal((Tk, Hk, D), 1.0, seed=900)
    vv = device_bf16_normal((Tk, Hk, D), 1.0, seed=901)
    ks = torch.empty(Hk, dtype=torch.float32, device=dev)
    vs = torch.empty(Hk, dtype=torch.float32, device=dev)
    kc = torch.empty((Tk, Hk, D), dtype=torch.uint8, device=dev)
    vc = torch.empty((Tk, Hk, D), dtype=torch.uint8, device=dev)
    slots = torch.arange(Tk, dtype=torch.int32, device=dev)
    for _ in range(R):
        fb.kv_scale_calibrate(kk, vv, True, ks, vs)
    torch.cuda.synchronize()
    for _ in range(R):
        fb.kv_cache_write_fp8(kk, vv, slots, ks, vs, kc, vc)
    del kk, vv, kc, vc
    done("kv")
    rb = rollout_batch(ROLLOUT_TRAIN_BATCH["responses"], ROLLOUT_TRAIN_BATCH["max_len"], (31, 1))
    lt, lr, adv = (torch.from_numpy(rb[key]).to(dev) for key in ("logp_train", "logp_rollout", "advantages"))
    msk = torch.from_numpy(rb["mask"]).to(dev)
    for _ in range(R):
        fb.token_importance_weights(lt, lr, C=2.0, mode="tis", mask=msk, advantages=adv)
    del lt, lr, adv, msk
    done("tis")
    w = device_bf16_normal((SWEEP_LAYERS, 24576, 4096), 0.02, seed=952)
    for _ in range(R):
        fb.quantize_weight_blockwise_dual(w)
    del w
    torch.cuda.synchronize()
    x = device_bf16_normal((PREFILL_M, 4096), 1.0, seed=960 + 4096)
    for _ in range(R):
        fb.quantize_act_dual(x)
    del x
    done("dual")


def bw_counter_summary(d):
    """Markdown table of the --bw-profile passes under `d` (kt, fetch, write,
    copy_fetch, copy_write): per case, the kernel's average duration, the HBM
    bytes per launch from FETCH_SIZE / WRITE_SIZE (copy-calibrated), the
    algorithmic bytes and their ratio, and the achieved fraction of 8 TB/s.
    Dispatches of the library's own kernels are matched to the cases in
    launch order (helper kernels such as the KV scale init are skipped)."""
    sys.path.insert(0, ROOT)
    from synthetic import ROLLOUT_TRAIN_BATCH, rollout_batch

    cases = bw_profile_cases()
    prefixes = {c[1] for c in cases}

    def ours(name):
        return any(re.search(r"\b%s\b" % re.escape(p), _short(name)) for p in prefixes)

    def dispatches(sub, key):
        out = {}
        pattern = "*kernel_trace.csv" if sub == "kt" else "*counter_collection.csv"
        for r in _csv_rows(os.path.join(d, sub, "**", pattern)):
            if ours(r["Kernel_Name"]):
                out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]}).update(key(r))
        return [out[i] for i in sorted(out)]

    kt = dispatches("kt", lambda r: {"ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
    fetch = dispatches("fetch", lambda r: {r["Counter_Name"]: float(r["Counter_Value"])})
    write = dispatches("write", lambda r: {r["Counter_Name"]: float(r["Counter_Value"])})
    scale = {"FETCH_SIZE": _copy_scale(d, "copy_fetch", "FETCH_SIZE"),
             "WRITE_SIZE": _copy_scale(d, "copy_write", "WRITE_SIZE")}
    rb = rollout_batch(ROLLOUT_TRAIN_BATCH["responses"], ROLLOUT_TRAIN_BATCH["max_len"], (31, 1))
    tis_bytes = importance_weight_bytes(rb["mask"].size, int(rb["mask"].sum()))
    n_expected = len(cases) * BW_PROFILE_REPS
    lines = ["Dispatches matched: kernel trace %d, fetch %d, write %d (expected %d).  Copy calibration: "
             "FETCH_SIZE x%s, WRITE_SIZE x%s." % (len(kt), len(fetch), len(write), n_expected,
                                                  "%.3f" % scale["FETCH_SIZE"] if scale["FETCH_SIZE"] else "n/a",
                                                  "%.3f" % scale["WRITE_SIZE"] if scale["WRITE_SIZE"] else "n/a"), "",
             "| case | kernel | us | HBM read / launch (MB) | HBM write / launch (MB) | measured / algorithmic MB "
             "| ratio | achieved GB/s (algorithmic) | frac of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]

    def avg(disp, c, key):
        if len(disp) != n_expected:
            return None
        xs = [x.get(key) for x in disp[c * BW_PROFILE_REPS:(c + 1) * BW_PROFILE_REPS]]
        xs = [x for x in xs if x is not None]
        return sum(xs) / len(xs) if xs else None

    for c, (label, prefix, algo) in enumerate(cases):
        algo = tis_bytes if algo is None else algo
        ns = avg(kt, c, "ns")
        fr = avg(fetch, c, "FETCH_SIZE")
        wr = avg(write, c, "WRITE_SIZE")
        name = _short(kt[c * BW_PROFILE_REPS]["name"]) if len(kt) == n_expected else "?"
        fb_ = fr * 1024.0 * scale["FETCH_SIZE"] if fr is not None and scale["FETCH_SIZE"] else None
        wb_ = wr * 1024.0 * scale["WRITE_SIZE"] if wr is not None and scale["WRITE_SIZE"] else None
        meas = fb_ + wb_ if fb_ is not None and wb_ is not None else None
        gbps = algo / ns if ns else None
        lines.append("| %s | `%s` | %s | %s | %s | %s | %s | %s | %s |" % (
            label, name[:70], "%.1f" % (ns / 1e3) if ns else "n/a",
            "%.1f" % (fb_ / 1e6) if fb_ is not None else "n/a", "%.1f" % (wb_ / 1e6) if wb_ is not None else "n/a",
            "%.1f / %.1f" % (meas / 1e6, algo / 1e6) if meas is not None else "n/a / %.1f" % (algo / 1e6),
            "%.3f" % (meas / algo) if meas is not None else "n/a", "%.0f" % gbps if gbps else "n/a",
            "%.3f" % (gbps / HBM_PEAK_GBPS) if gbps else "n/a"))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
