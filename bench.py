"""Benchmark of the blockwise W8A8 FP8 hot path on one MI355X.

One step = the whole linear-layer hot path for a Qwen3-8B-shaped decode
layer (M = 256 tokens): re-quantize the four BF16 weight matrices (qkv
4096->6144, o 4096->4096, gate_up 4096->24576, down 12288->4096) into E4M3
with 128x128-block FP32 scales, quantize the four BF16 activations per token
in 1x128 groups, and run the four block-scaled FP8 GEMMs (FP32 accumulation,
BF16 output).  Inputs are seeded synthetic tensors already resident in HBM.

`value` = W8A8 GEMM FLOPs of the step / step time (TFLOP/s, the re-quant
and activation quantization inside the timed step).  The JSON line adds the
roofline of the dominant kernel (the weight re-quantizer, timed with HIP
events on its stream inside the timed region), the CPU oracle timed on a
bounded sample, and per-configuration details measured after the timed
region: prefill GEMMs (M = 8192), the MoE grouped GEMMs, the 36-layer
re-quantization sweep, and sampled parity against the oracle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-detail] [--no-cpu]
       python bench.py --rocprof-summary DIR   (summarise rocprofv3 output, see below)

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
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_layer_step_qwen3_8b.md")
# kernel-name prefix of each phase -> the source file that defines it
# launches per decode step: the four matrices are re-quantized by one launch
PHASE_LAUNCHES = {"requant": 1, "act_quant": 4, "gemm": 4}
PHASE_KERNELS = {
    "requant": ("quant_weight_multi_kernel", "quant.hip"),
    "act_quant": ("quant_act_kernel", "quant.hip"),
    "gemm": ("gemm_dense_kernel", "gemm.hip"),
}


def source_sha(fname):
    """SHA-256 of a kernel source plus every shared device header."""
    h = hashlib.sha256()
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".hpp"))
    for f in (fname, *headers):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
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
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-detail", action="store_true", help="skip the per-configuration measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale HBM byte counters) and exit")
    p.add_argument("--rocprof-summary", metavar="DIR",
                   help="summarise rocprofv3 output under DIR (kernel trace + FETCH_SIZE / WRITE_SIZE passes "
                        "of this benchmark and of --calibrate-copy) and exit")
    p.add_argument("--gemm-profile", action="store_true",
                   help="only run each GEMM of GEMM_PROFILE_CASES a few times (a target for rocprofv3 "
                        "counter passes) and exit")
    p.add_argument("--gemm-counter-summary", metavar="DIR",
                   help="summarise rocprofv3 passes of --gemm-profile under DIR (kt, mfma, lds, l2, fetch, "
                        "write, copy_fetch, copy_write) and exit")
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
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path.  Its kernels run on "
              "one GPU's share of the work: whole 128x128 weight blocks for re-quantization, column- or "
              "row-parallel GEMM slices at multiples of 128, or whole experts.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import fp8_blockwise_quantized_quantize_amd as fb
    from synthetic import LAYER_SHAPES_QWEN3_8B, device_bf16_normal

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    M = 256

    # ---------------------------------------------------------------- inputs
    # Step s uses buffer set s % SETS (copies of the same inputs): one set is
    # ~0.6 GB, so a set has left the 256 MB Infinity Cache before it is used
    # again and the step's weight bytes come from HBM.
    SETS = 4
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
    layers = sets[0]
    gemm_flops = sum(2 * M * L["n"] * L["k"] for L in layers)
    requant_bytes = sum(L["n"] * L["k"] * 3 + L["ws"].numel() * 4 for L in layers)

    # HIP events between the three phases of a step, on the launch stream
    phases = ("requant", "act_quant", "gemm")
    ev = []

    def step(record, s):
        ls = sets[s % SETS]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        # the layer's four matrices re-quantized by one launch
        fb.quantize_weights_blockwise_multi([L["w"] for L in ls], [(L["wq"], L["ws"]) for L in ls])
        if record:
            e[1].record(stream)
        for L in ls:
            fb.quantize_act_per_token_group(L["x"], L["xq"], L["xs"])
        if record:
            e[2].record(stream)
        for L in ls:
            fb.gemm_w8a8_blockscaled(L["xq"], L["xs"], L["wq"], L["ws"], L["y"])
        if record:
            e[3].record(stream)
            ev.append(e)

    for s in range(args.warmup):
        step(False, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(True, s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step(False, 0)  # set 0 holds this step's outputs for the parity check below
    torch.cuda.synchronize()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # per-phase time (ms per step) and algorithmic bytes / FLOPs per step
    phase_ms = {p: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / len(ev) for i, p in enumerate(phases)}
    act_bytes = sum(M * L["k"] * 3 + L["xs"].numel() * 4 for L in layers)
    gemm_bytes = sum(M * L["k"] + L["n"] * L["k"] + 2 * M * L["n"] + L["xs"].numel() * 4 + L["ws"].numel() * 4
                     for L in layers)
    kernels = {
        "requant": (PHASE_KERNELS["requant"][0], requant_bytes, 0),
        "act_quant": (PHASE_KERNELS["act_quant"][0], act_bytes, 0),
        "gemm": (PHASE_KERNELS["gemm"][0], gemm_bytes, gemm_flops),
    }
    roof_all = {}
    for p in phases:
        name, byt, flops = kernels[p]
        ms = phase_ms[p]
        nl = PHASE_LAUNCHES[p]
        launch_us = ms * 1e3 / nl
        # bound: HBM unless the arithmetic intensity passes the ridge point
        if flops and flops / byt > FP8_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3:
            ach, peak, unit, bound = flops / ms / 1e9, FP8_PEAK_TFLOPS, "TFLOP/s", "mfma"
        else:
            ach, peak, unit, bound = byt / ms / 1e6, HBM_PEAK_GBPS, "GB/s", "hbm"
        tr = committed_traffic(p)
        roof_all[p] = {"bound": bound, "kernel": name, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                       "frac": round(ach / peak, 4), "traffic": tr["bytes_per_launch"] if tr else None,
                       "avg_launch_us": round(launch_us, 2),
                       "launches_per_step": nl, "algorithmic_bytes_per_launch_avg": int(byt / nl),
                       "flops_per_launch_avg": int(flops / nl)}
        if flops:
            roof_all[p]["TFLOPs"] = round(flops / ms / 1e9, 1)
    dominant = max(phases, key=lambda p: phase_ms[p])
    roofline = dict(roof_all[dominant])
    requant_gbps = requant_bytes / phase_ms["requant"] / 1e6

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
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; Qwen3-8B layer shapes; "
                "4 buffer sets rotated across steps)",
        "config": {
            "workload": "qwen3-8b-decode-layer: requant qkv/o/gate_up/down + 1x128 act quant + 4 W8A8 GEMMs, M=256",
            "tokens": M,
            "gemm_flops_per_step": gemm_flops,
            "requant_bytes_per_step": requant_bytes,
            "parallelism": "1 GPU",
        },
        "roofline": roofline,
        "roofline_per_kernel": roof_all,
        "phase_ms": {p: round(v, 4) for p, v in phase_ms.items()},
        "requant_GBps": round(requant_gbps, 1),
        "requant_frac_hbm": round(requant_gbps / HBM_PEAK_GBPS, 4),
        "device": device_info(),
    }

    if not args.no_detail:
        out["detail"] = detail(fb, dev)
    if not args.no_cpu:
        out["cpu_baseline"], out["parity"] = cpu_baseline(layers, M, gemm_flops, requant_bytes)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# Per-configuration measurements (after the timed region)
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


def detail(fb, dev):
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B, device_bf16_normal, moe_routing

    res = {}
    # -- prefill GEMMs, M = 8192, activations with 1% outlier channels x30
    m = 8192
    pre = {}
    tot_f = tot_ms = tot_fr_ms = 0.0
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((n, k), 0.02, seed=300 + i)
        x = device_bf16_normal((m, k), 1.0, seed=400 + i)
        g = torch.Generator().manual_seed(500 + i)
        cols = torch.randperm(k, generator=g)[: round(0.01 * k)].to(dev)
        x[:, cols] = (x[:, cols].float() * 30.0).to(torch.bfloat16)
        wq, ws = fb.quantize_weight_blockwise(w)
        xq, xs = fb.quantize_act_per_token_group(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms, ms_min = _time_graph_ms(lambda: fb.gemm_w8a8_blockscaled(xq, xs, wq, ws, y), calls=4)
        # the same GEMM on fragment-order activation codes (same result bits)
        xf, _ = fb.quantize_act_per_token_group_frag(x)
        fr_ms, _ = _time_graph_ms(lambda: fb.gemm_w8a8_blockscaled_afrag(xf, xs, wq, ws, y), calls=4)
        del xf
        sets = [(x, xq, xs)] + [(x.clone(), torch.empty_like(xq), torch.empty_like(xs))
                                for _ in range(rotations(m * k * 3) - 1)]
        aq_ms, _ = _time_graph_ms([lambda t=t: fb.quantize_act_per_token_group(*t) for t in sets])
        aqf_ms, _ = _time_graph_ms([lambda t=t: fb.quantize_act_per_token_group_frag(*t) for t in sets])
        del sets
        f = 2 * m * n * k
        tot_f += f
        tot_ms += ms
        tot_fr_ms += fr_ms
        pre[name] = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(f / ms / 1e9, 1),
                     "frac_fp8_peak": round(f / ms / 1e9 / FP8_PEAK_TFLOPS, 4),
                     "afrag_gemm_us": round(fr_ms * 1e3, 1), "afrag_TFLOPs": round(f / fr_ms / 1e9, 1),
                     "afrag_frac_fp8_peak": round(f / fr_ms / 1e9 / FP8_PEAK_TFLOPS, 4),
                     "act_quant_us": round(aq_ms * 1e3, 1), "afrag_act_quant_us": round(aqf_ms * 1e3, 1),
                     "act_quant_GBps": round((m * k * 3 + m * (k // 128) * 4) / aq_ms / 1e6, 1)}
        del w, x, wq, ws, xq, xs, y
    pre["all4"] = {"TFLOPs": round(tot_f / tot_ms / 1e9, 1), "frac_fp8_peak": round(tot_f / tot_ms / 1e9 / FP8_PEAK_TFLOPS, 4),
                   "afrag_TFLOPs": round(tot_f / tot_fr_ms / 1e9, 1),
                   "afrag_frac_fp8_peak": round(tot_f / tot_fr_ms / 1e9 / FP8_PEAK_TFLOPS, 4)}
    res["prefill_gemm_M8192"] = pre
    torch.cuda.empty_cache()

    # -- one MoE expert-FFN layer (Qwen3-30B-A3B: 4096 tokens, top-8 of 128
    #    experts, hidden 2048, expert FFN 768), every step on the GPU:
    #    sort -> 1x128 quant of the tokens -> fc1 (rows gathered by routed pair)
    #    -> SiLU*up + 1x128 quant -> fc2 -> combine
    res["moe_layer_qwen3_30b_a3b"] = moe_layer(fb, dev)
    torch.cuda.empty_cache()

    # -- 36-layer re-quantization sweep (4 calls, batch = 36 each)
    sweep_bytes = 0
    bufs = []
    for p, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((36, n, k), 0.02, seed=800 + p)
        q = torch.empty((36, n, k), dtype=torch.uint8, device=dev)
        s = torch.empty((36, n // 128, k // 128), dtype=torch.float32, device=dev)
        bufs.append((w, q, s))
        sweep_bytes += 36 * n * k * 3 + s.numel() * 4

    def sweep():
        for w, q, s in bufs:
            fb.quantize_weight_blockwise(w, q, s)

    ms, ms_min = _time_ms(sweep, reps=5, warm=1)
    gbps = sweep_bytes / ms / 1e6
    res["requant_sweep_36_layers"] = {"params": sum(w.numel() for w, _, _ in bufs), "bytes": sweep_bytes,
                                      "ms": round(ms, 3), "GBps": round(gbps, 1),
                                      "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
    del bufs
    torch.cuda.empty_cache()

    # -- FP8 training operands (Qwen3-8B): W and W^T of all 36 layers' four
    #    projections, and x / x^T of an 8192-token micro-batch's layer inputs
    res["train_operands_qwen3_8b"] = train_operands(fb, dev)
    torch.cuda.empty_cache()

    # -- FP8 KV cache, one Qwen3-8B layer (8 KV heads x 128): a rollout's first
    #    forward calibrates the per-head scales on a 16384-token prefill chunk
    #    and writes it to the cache; a decode step then writes 1536 tokens
    res["kv_cache_qwen3_8b_layer"] = kv_cache(fb, dev)
    torch.cuda.empty_cache()

    # -- token-level TIS weights of one training batch (512 responses padded
    #    to 20,000 tokens), fused with the response mask and w * advantage
    from synthetic import ROLLOUT_TRAIN_BATCH, rollout_batch

    rb = rollout_batch(ROLLOUT_TRAIN_BATCH["responses"], ROLLOUT_TRAIN_BATCH["max_len"], (31, 1))
    lt, lr, adv = (torch.from_numpy(rb[k]).to(dev) for k in ("logp_train", "logp_rollout", "advantages"))
    msk = torch.from_numpy(rb["mask"]).to(dev)
    slots, valid = lt.numel(), int(rb["mask"].sum())
    byt = importance_weight_bytes(slots, valid)
    sets = [(t.clone() for t in (lt, lr, msk, adv)) for _ in range(rotations(21 * slots))]
    sets = [tuple(g) + (torch.empty_like(lt), torch.empty_like(lt)) for g in sets]
    ms, ms_min = _time_graph_ms([lambda t=t: fb.token_importance_weights(t[0], t[1], C=2.0, mode="tis", mask=t[2],
                                                                         advantages=t[3], out=t[4], out_adv=t[5])
                                 for t in sets])
    del sets
    gbps = byt / ms / 1e6
    res["tis_weights_train_batch_512x20000"] = {"tokens": valid, "slots": slots, "bytes": byt,
                                                "us": round(ms * 1e3, 1), "GBps": round(gbps, 1),
                                                "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
    del lt, lr, adv, msk
    torch.cuda.empty_cache()
    return res


def moe_layer(fb, dev):
    import torch

    from synthetic import MOE_QWEN3_30B_A3B, device_bf16_normal, moe_topk

    cfg = MOE_QWEN3_30B_A3B
    T, E, k, H, F = cfg["tokens"], cfg["experts"], cfg["top_k"], cfg["hidden"], cfg["ffn"]
    R = T * k
    ids_h, tw_h = moe_topk(T, E, k, (70, 0))
    ids, tw = torch.from_numpy(ids_h).to(dev), torch.from_numpy(tw_h).to(dev)
    x = device_bf16_normal((T, H), 1.0, seed=700)
    w1q, w1s = fb.quantize_weight_blockwise(device_bf16_normal((E, 2 * F, H), 0.02, seed=600))
    w2q, w2s = fb.quantize_weight_blockwise(device_bf16_normal((E, H, F), 0.02, seed=601))
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
    steps = {
        "sort": ([lambda: fb.moe_sort_by_expert(ids, E, off, sp, pr)], None, None),
        "act_quant": ([lambda t=t: fb.quantize_act_per_token_group(*t) for t in aq_sets], aq_b, None),
        "fc1_gate_up": ([lambda t=t: fb.grouped_gemm_w8a8_blockscaled_gather(a, a_s, sp, k, t[0], t[1], off, t[2])
                         for t in w1_sets], None, 2 * R * 2 * F * H),
        "silu_mul_quant": ([lambda t=t: fb.silu_mul_quantize_act(*t) for t in silu_sets], silu_b, None),
        "fc2_down": ([lambda t=t: fb.grouped_gemm_w8a8_blockscaled(h, h_s, t[0], t[1], off, t[2]) for t in w2_sets],
                     None, 2 * R * H * F),
        "combine": ([lambda t=t: fb.moe_combine(t[0], pr, tw, t[1]) for t in comb_sets], comb_b, None),
    }
    res, total = {}, 0.0
    for name, (fn, byt, flops) in steps.items():
        ms, _ = _time_graph_ms(fn)
        e_rot = len(fn)
        total += ms
        e = {"us": round(ms * 1e3, 1), "buffer_sets": e_rot}
        if byt is not None:
            e.update({"bytes": byt, "GBps": round(byt / ms / 1e6, 1), "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBPS, 4)})
        if flops is not None:
            n_out = 2 * F if name == "fc1_gate_up" else H
            k_in = H if name == "fc1_gate_up" else F
            a_rows = T if name == "fc1_gate_up" else R  # fc1 reads each token's row once (gathered)
            byt_g = a_rows * k_in + E * n_out * k_in + 2 * R * n_out + a_rows * (k_in // 128) * 4
            roof = min(FP8_PEAK_TFLOPS, flops / byt_g * HBM_PEAK_GBPS / 1e3)
            e.update({"TFLOPs": round(flops / ms / 1e9, 1), "roofline_TFLOPs": round(roof, 1),
                      "frac_roofline": round(flops / ms / 1e9 / roof, 4)})
        res[name] = e

    def layer():
        fb.moe_expert_ffn(x, ids, tw, w1q, w1s, w2q, w2s)

    layer_ms, _ = _time_graph_ms(layer, calls=4)
    del aq_sets, w1_sets, silu_sets, w2_sets, comb_sets
    res["sum_of_kernels_us"] = round(total * 1e3, 1)
    res["layer_us"] = round(layer_ms * 1e3, 1)
    res["layer_TFLOPs"] = round((2 * R * 2 * F * H + 2 * R * H * F) / layer_ms / 1e9, 1)
    return res


def train_operands(fb, dev):
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

    ms, _ = _time_ms(sweep, reps=3, warm=1)
    res["weight_dual_sweep_36_layers"] = {"bytes": wbytes, "ms": round(ms, 3), "GBps": round(wbytes / ms / 1e6, 1),
                                          "frac_hbm": round(wbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
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
        del x
    return res


def kv_cache(fb, dev):
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
    return res


def importance_weight_bytes(slots, valid):
    """Algorithmic HBM bytes of the fused importance-weight pass: the two
    log-probs and the advantage of each generated token (12 B), the mask byte
    and the two float32 outputs of every slot, padding included (9 B)."""
    return 12 * valid + 9 * slots


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample, with parity of that sample
# ---------------------------------------------------------------------------

def cpu_baseline(layers, m, gemm_flops, requant_bytes):
    """Time the oracle on one whole decode-layer step and check the GPU's
    results of the timed run against it.

    The oracle runs the same step on the same input bytes: re-quantization
    of the four weight matrices (193M parameters, numpy), the four per-token
    activation quantizations, and the four GEMMs through its float64 path
    (BLAS matmul).  It is untuned test infrastructure; the figure is a
    reported baseline, not a target.
    """
    import torch

    import oracle
    from oracle import gemm_ref, quant_act_per_token_group, quant_weight_blockwise

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    host = [(bits(L["w"]), bits(L["x"])) for L in layers]
    t0 = time.perf_counter()
    wres = [quant_weight_blockwise(w) for w, _ in host]
    t_rq = time.perf_counter() - t0
    t0 = time.perf_counter()
    ares = [quant_act_per_token_group(x) for _, x in host]
    t_aq = time.perf_counter() - t0
    t0 = time.perf_counter()
    yres = [gemm_ref(qa, sa, qw, sw) for (qa, sa), (qw, sw) in zip(ares, wres)]
    t_gm = time.perf_counter() - t0
    total = t_rq + t_aq + t_gm
    cores = len(os.sched_getaffinity(0))
    base = {
        "value": round(gemm_flops / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": ("one full decode-layer step (4 weight re-quants, 193M params, numpy single-threaded; 4 activation "
                   "quants; 4 GEMMs as float64 BLAS matmuls on %d threads), same input bytes as the GPU run" % cores),
        "seconds": {"requant": round(t_rq, 3), "act_quant": round(t_aq, 3), "gemm": round(t_gm, 3)},
        "requant_GBps": round(requant_bytes / t_rq / 1e9, 3),
    }

    par = {"requant_bitexact": True, "act_quant_bitexact": True, "gemm": {}}
    for L, (qw, sw), (qa, sa), y_ref in zip(layers, wres, ares, yres):
        par["requant_bitexact"] &= bool(np.array_equal(L["wq"].cpu().numpy(), qw) and np.array_equal(
            L["ws"].cpu().numpy().view(np.uint32), sw.view(np.uint32)))
        par["act_quant_bitexact"] &= bool(np.array_equal(L["xq"].cpu().numpy(), qa) and np.array_equal(
            L["xs"].cpu().numpy().view(np.uint32), sa.view(np.uint32)))
        y = L["y"].view(torch.int16).cpu().numpy().view(np.uint16)
        yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rel_fro = float(np.linalg.norm(yf - y_ref) / np.linalg.norm(y_ref))
        rms = float(np.sqrt(np.mean(y_ref ** 2)))
        rel_max = float(np.max(np.abs(yf - y_ref) / np.maximum(np.abs(y_ref), rms)))
        exact = float(np.mean(y == oracle.round_to_bf16_bits(y_ref)))
        par["gemm"][L["name"]] = {"rel_fro": round(rel_fro, 6), "rel_max": round(rel_max, 6),
                                  "exact_bf16_frac": round(exact, 4), "pass": rel_fro <= 1e-2 and rel_max <= 1e-2}
    return base, par


# ---------------------------------------------------------------------------
# rocprofv3 summary (kernel trace + HBM byte counters)
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
        if prefix in kernel_name:
            return p
    return None


def step_algorithmic_bytes(M=256):
    """Average algorithmic HBM bytes per launch of each phase of the decode step."""
    sys.path.insert(0, ROOT)
    from synthetic import LAYER_SHAPES_QWEN3_8B

    rq = aq = gm = 0
    for _, n, k in LAYER_SHAPES_QWEN3_8B:
        ws = (n // 128) * (k // 128) * 4
        xs = M * (k // 128) * 4
        rq += n * k * 3 + ws
        aq += M * k * 3 + xs
        gm += M * k + n * k + 2 * M * n + xs + ws
    return {"requant": rq / PHASE_LAUNCHES["requant"], "act_quant": aq / PHASE_LAUNCHES["act_quant"],
            "gemm": gm / PHASE_LAUNCHES["gemm"]}


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

    copy_bytes = float(1 << 30)
    scale = {}
    for sub, counter in (("copy_fetch", "FETCH_SIZE"), ("copy_write", "WRITE_SIZE")):
        v = [x for name, xs in per_dispatch(sub, counter).items() if "copyBuffer" in name for x in xs]
        scale[counter] = copy_bytes / (sum(v) / len(v)) if v else None
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
    lines.append("| phase (decode step) | measured HBM bytes / launch (MB) | algorithmic bytes / launch (MB) | ratio |")
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

    cases = [("decode %s" % nm, 256, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    cases += [("prefill %s" % nm, 8192, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    cases += [("prefill afrag %s" % nm, 8192, n, k, 0) for nm, n, k in LAYER_SHAPES_QWEN3_8B]
    moe = MOE_QWEN3_30B_A3B
    mt = moe["tokens"] * moe["top_k"]
    cases.append(("MoE fc1 gate_up", mt, moe["gate_up"][0], moe["gate_up"][1], moe["experts"]))
    cases.append(("MoE fc2 down", mt, moe["down"][0], moe["down"][1], moe["experts"]))
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
        wq, ws = fb.quantize_weight_blockwise(w)
        afrag = label.startswith("prefill afrag")
        if afrag:
            xq, xs = fb.quantize_act_per_token_group_frag(x)
        else:
            xq, xs = fb.quantize_act_per_token_group(x)
        del w, x
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        torch.cuda.synchronize()
        for _ in range(GEMM_PROFILE_REPS):
            if afrag:
                fb.gemm_w8a8_blockscaled_afrag(xq, xs, wq, ws, y)
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
      fetch / write, copy_fetch / copy_write   as for the decode-step summary
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

    copy = {}
    for sub, counter in (("copy_fetch", "FETCH_SIZE"), ("copy_write", "WRITE_SIZE")):
        v = [float(r["Counter_Value"]) * 1024.0
             for r in _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv"))
             if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
        copy[counter] = float(1 << 30) / (sum(v) / len(v)) if v else None
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
        algo = m * k + (g or 1) * n * k + 2 * m * n + 4 * m * (k // 128) + 4 * (g or 1) * nb * (k // 128)
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


if __name__ == "__main__":
    main()
