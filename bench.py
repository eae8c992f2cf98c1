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
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-detail", action="store_true", help="skip the per-configuration measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the kernels run on one GPU's share of the work; see DESIGN.md for how it would shard).",
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
    layers = []
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((n, k), 0.02, seed=100 + i)
        x = device_bf16_normal((M, k), 1.0, seed=200 + i)
        layers.append({
            "name": name, "n": n, "k": k, "w": w, "x": x,
            "wq": torch.empty((n, k), dtype=torch.uint8, device=dev),
            "ws": torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev),
            "xq": torch.empty((M, k), dtype=torch.uint8, device=dev),
            "xs": torch.empty((M, k // 128), dtype=torch.float32, device=dev),
            "y": torch.empty((M, n), dtype=torch.bfloat16, device=dev),
        })
    gemm_flops = sum(2 * M * L["n"] * L["k"] for L in layers)
    requant_bytes = sum(L["n"] * L["k"] * 3 + L["ws"].numel() * 4 for L in layers)

    ev = []  # (start, end) HIP events around the re-quantizer launches

    def step(record):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        for L in layers:
            fb.quantize_weight_blockwise(L["w"], L["wq"], L["ws"])
        if record:
            e1.record(stream)
            ev.append((e0, e1))
        for L in layers:
            fb.quantize_act_per_token_group(L["x"], L["xq"], L["xs"])
            fb.gemm_w8a8_blockscaled(L["xq"], L["xs"], L["wq"], L["ws"], L["y"])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    requant_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)  # 4 launches per step
    requant_launch_ms = requant_ms / len(layers)
    requant_gbps = requant_bytes / (requant_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "quant_weight_kernel",
        "achieved": round(requant_gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(requant_gbps / HBM_PEAK_GBPS, 4),
        "traffic": None,
        "avg_launch_us": round(requant_launch_ms * 1e3, 2),
        "bytes_per_launch_avg": int(requant_bytes / len(layers)),
    }

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
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; Qwen3-8B layer shapes)",
        "config": {
            "workload": "qwen3-8b-decode-layer: requant qkv/o/gate_up/down + 1x128 act quant + 4 W8A8 GEMMs, M=256",
            "tokens": M,
            "gemm_flops_per_step": gemm_flops,
            "requant_bytes_per_step": requant_bytes,
            "parallelism": "1 GPU",
        },
        "roofline": roofline,
        "requant_GBps": round(requant_gbps, 1),
        "requant_frac_hbm": round(requant_gbps / HBM_PEAK_GBPS, 4),
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


def detail(fb, dev):
    import torch

    from synthetic import LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B, device_bf16_normal, moe_routing

    res = {}
    # -- prefill GEMMs, M = 8192, activations with 1% outlier channels x30
    m = 8192
    pre = {}
    tot_f = tot_ms = 0.0
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        w = device_bf16_normal((n, k), 0.02, seed=300 + i)
        x = device_bf16_normal((m, k), 1.0, seed=400 + i)
        g = torch.Generator().manual_seed(500 + i)
        cols = torch.randperm(k, generator=g)[: round(0.01 * k)].to(dev)
        x[:, cols] = (x[:, cols].float() * 30.0).to(torch.bfloat16)
        wq, ws = fb.quantize_weight_blockwise(w)
        xq, xs = fb.quantize_act_per_token_group(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms, ms_min = _time_ms(lambda: fb.gemm_w8a8_blockscaled(xq, xs, wq, ws, y), reps=10)
        aq_ms, _ = _time_ms(lambda: fb.quantize_act_per_token_group(x, xq, xs), reps=10)
        f = 2 * m * n * k
        tot_f += f
        tot_ms += ms
        pre[name] = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(f / ms / 1e9, 1),
                     "frac_fp8_peak": round(f / ms / 1e9 / FP8_PEAK_TFLOPS, 4),
                     "act_quant_us": round(aq_ms * 1e3, 1),
                     "act_quant_GBps": round((m * k * 3 + m * (k // 128) * 4) / aq_ms / 1e6, 1)}
        del w, x, wq, ws, xq, xs, y
    pre["all4"] = {"TFLOPs": round(tot_f / tot_ms / 1e9, 1), "frac_fp8_peak": round(tot_f / tot_ms / 1e9 / FP8_PEAK_TFLOPS, 4)}
    res["prefill_gemm_M8192"] = pre
    torch.cuda.empty_cache()

    # -- MoE grouped GEMMs (Qwen3-30B-A3B layer, 4096 tokens, top-8 of 128)
    cfg = MOE_QWEN3_30B_A3B
    tok, _, off = moe_routing(cfg["tokens"], cfg["experts"], cfg["top_k"], (70, 0))
    offd = torch.from_numpy(off).to(dev)
    mt = int(off[-1])
    moe = {}
    for j, proj in enumerate(("gate_up", "down")):
        n, k = cfg[proj]
        w = device_bf16_normal((cfg["experts"], n, k), 0.02, seed=600 + j)
        x = device_bf16_normal((mt, k), 1.0, seed=700 + j)
        wq, ws = fb.quantize_weight_blockwise(w)
        xq, xs = fb.quantize_act_per_token_group(x)
        y = torch.empty((mt, n), dtype=torch.bfloat16, device=dev)
        ms, _ = _time_ms(lambda: fb.grouped_gemm_w8a8_blockscaled(xq, xs, wq, ws, offd, y), reps=10)
        f = 2 * mt * n * k
        byt = mt * k + cfg["experts"] * n * k + 2 * mt * n + xs.numel() * 4 + ws.numel() * 4
        roof = min(FP8_PEAK_TFLOPS, f / byt * HBM_PEAK_GBPS / 1e3)
        moe[proj] = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(f / ms / 1e9, 1),
                     "roofline_TFLOPs": round(roof, 1), "frac_roofline": round(f / ms / 1e9 / roof, 4)}
        del w, x, wq, ws, xq, xs, y
    res["moe_grouped"] = moe
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
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample, with parity of that sample
# ---------------------------------------------------------------------------

def cpu_baseline(layers, m, gemm_flops, requant_bytes):
    """Time the oracle on part of the decode-layer step and check the GPU's
    results for that part against it.

    Sample: re-quantization of the o projection (4096 x 4096), activation
    quantization of all four inputs (256 x 4096 x 3, 256 x 12288), and the
    o-projection GEMM (256 x 4096 x 4096) through the oracle's float64 path.
    The step time is extrapolated by parameters (re-quant) and FLOPs (GEMM).
    """
    import torch

    import oracle
    from oracle import gemm_ref, quant_act_per_token_group, quant_weight_blockwise

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    o = next(L for L in layers if L["name"] == "o")
    w_bits = bits(o["w"])
    t0 = time.perf_counter()
    oq, os_ = quant_weight_blockwise(w_bits)
    t_rq = time.perf_counter() - t0
    acts = []
    t0 = time.perf_counter()
    for L in layers:
        acts.append(quant_act_per_token_group(bits(L["x"])))
    t_aq = time.perf_counter() - t0
    o_idx = [L["name"] for L in layers].index("o")
    qa, sa = acts[o_idx]
    t0 = time.perf_counter()
    y_ref = gemm_ref(qa, sa, oq, os_)
    yb_ref = oracle.round_to_bf16_bits(y_ref)
    t_gm = time.perf_counter() - t0

    params = sum(L["n"] * L["k"] for L in layers)
    o_flops = 2 * m * o["n"] * o["k"]
    est = t_rq * params / (o["n"] * o["k"]) + t_aq + t_gm * gemm_flops / o_flops
    cores = len(os.sched_getaffinity(0))
    base = {
        "value": round(gemm_flops / est / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": ("o-proj 4096x4096 re-quant (numpy, 1 thread), 4 activation quants, o-proj GEMM 256x4096x4096 "
                   "(float64 BLAS, %d threads); step time extrapolated by params and FLOPs" % cores),
        "sample_seconds": round(t_rq + t_aq + t_gm, 2),
        "est_step_s": round(est, 3),
        "requant_GBps": round(requant_bytes / (t_rq * params / (o["n"] * o["k"])) / 1e9, 3),
    }

    # parity of the sampled part
    par = {}
    par["requant_o_bitexact"] = bool(np.array_equal(o["wq"].cpu().numpy(), oq)
                                     and np.array_equal(o["ws"].cpu().numpy().view(np.uint32), os_.view(np.uint32)))
    ok = True
    for L, (q, s) in zip(layers, acts):
        ok &= bool(np.array_equal(L["xq"].cpu().numpy(), q)
                   and np.array_equal(L["xs"].cpu().numpy().view(np.uint32), s.view(np.uint32)))
    par["act_quant_bitexact"] = ok
    y = o["y"].view(torch.int16).cpu().numpy().view(np.uint16)
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel_fro = float(np.linalg.norm(yf - y_ref) / np.linalg.norm(y_ref))
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    rel_max = float(np.max(np.abs(yf - y_ref) / np.maximum(np.abs(y_ref), rms)))
    par["gemm_o"] = {"rel_fro": rel_fro, "rel_max": rel_max, "exact_bf16_frac": float(np.mean(y == yb_ref)),
                     "pass": rel_fro <= 1e-2 and rel_max <= 1e-2}
    return base, par


if __name__ == "__main__":
    main()
