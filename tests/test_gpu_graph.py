"""The library's kernels under HIP graph capture: a decode-layer step
(re-quant, activation quant, GEMMs) in row-major and in fragment order
(one-launch quantizers, the fragment-order GEMM), a ragged MoE grouped GEMM
(plain and with gathered rows; the persistent expert-tile kernel by
default), the fragment-order activation quantizer with the activation-only
fragment GEMM, and a KV-cache calibration + write are
captured once and replayed several times, with eager work and
synchronizations between replays; every replay's outputs must equal the
eager outputs bit for bit (the kernels are deterministic and no memset is
captured)."""

import numpy as np
import pytest

from helpers import announce

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def snapshot(ts):
    torch.cuda.synchronize()
    return [t.clone() for t in ts]


def test_graph_replays_match_eager():
    from synthetic import LAYER_SHAPES_QWEN3_8B, device_bf16_normal

    M = 256
    layers = []
    for i, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B[:2]):
        layers.append(dict(w=device_bf16_normal((n, k), 0.02, seed=40 + i), x=device_bf16_normal((M, k), 1.0, seed=50 + i),
                           wq=torch.empty((n, k), dtype=torch.uint8, device=DEV),
                           ws=torch.empty((n // 128, k // 128), dtype=torch.float32, device=DEV),
                           xq=torch.empty((M, k), dtype=torch.uint8, device=DEV),
                           xs=torch.empty((M, k // 128), dtype=torch.float32, device=DEV),
                           y=torch.empty((M, n), dtype=torch.bfloat16, device=DEV)))
    H, D, T = 8, 128, 1000
    kv = dict(k=device_bf16_normal((T, H, D), 1.0, seed=60), v=device_bf16_normal((T, H, D), 1.0, seed=61),
              ks=torch.empty(H, dtype=torch.float32, device=DEV), vs=torch.empty(H, dtype=torch.float32, device=DEV),
              kc=torch.zeros((T, H, D), dtype=torch.uint8, device=DEV),
              vc=torch.zeros((T, H, D), dtype=torch.uint8, device=DEV),
              slots=torch.arange(T, dtype=torch.int32, device=DEV))

    G, NE, KE = 16, 256, 384
    counts = np.array([0, 37, 300, 1, 0, 129, 256, 3, 0, 90, 17, 400, 2, 0, 64, 5], np.int64)
    Me = int(counts.sum())
    moe = dict(wq=torch.empty((G, NE, KE), dtype=torch.uint8, device=DEV),
               ws=torch.empty((G, NE // 128, KE // 128), dtype=torch.float32, device=DEV),
               xq=torch.empty((Me, KE), dtype=torch.uint8, device=DEV),
               xs=torch.empty((Me, KE // 128), dtype=torch.float32, device=DEV),
               off=torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=DEV),
               rows=torch.tensor(np.random.default_rng(7).integers(-1, 2 * Me, Me).astype(np.int32), device=DEV),
               y=torch.empty((Me, NE), dtype=torch.bfloat16, device=DEV),
               yg=torch.empty((Me, NE), dtype=torch.bfloat16, device=DEV))
    fb().quantize_weight_blockwise(device_bf16_normal((G, NE, KE), 0.02, seed=70), moe["wq"], moe["ws"])
    fb().quantize_act_per_token_group(device_bf16_normal((Me, KE), 1.0, seed=71), moe["xq"], moe["xs"])

    L0 = layers[0]
    af = dict(xq=torch.empty_like(L0["xq"]), xs=torch.empty_like(L0["xs"]), y=torch.empty_like(L0["y"]))
    fr = [dict(wq=torch.empty_like(L["wq"]), ws=torch.empty_like(L["ws"]), xq=torch.empty_like(L["xq"]),
               xs=torch.empty_like(L["xs"]), y=torch.empty_like(L["y"])) for L in layers]

    def work():
        fb().grouped_gemm_w8a8_blockscaled(moe["xq"], moe["xs"], moe["wq"], moe["ws"], moe["off"], moe["y"])
        fb().grouped_gemm_w8a8_blockscaled_gather(moe["xq"], moe["xs"], moe["rows"], 2, moe["wq"], moe["ws"],
                                                  moe["off"], moe["yg"])
        for L in layers:
            fb().quantize_weight_blockwise(L["w"], L["wq"], L["ws"])
            fb().quantize_act_per_token_group(L["x"], L["xq"], L["xs"])
            fb().gemm_w8a8_blockscaled(L["xq"], L["xs"], L["wq"], L["ws"], L["y"])
        fb().quantize_act_per_token_group_frag(L0["x"], af["xq"], af["xs"])
        fb().gemm_w8a8_blockscaled_afrag(af["xq"], af["xs"], L0["wq"], L0["ws"], af["y"])
        fb().quantize_weights_blockwise_frag_multi([L["w"] for L in layers], [(F["wq"], F["ws"]) for F in fr])
        fb().quantize_acts_per_token_group_frag_multi([L["x"] for L in layers], [(F["xq"], F["xs"]) for F in fr])
        for F in fr:
            fb().gemm_w8a8_blockscaled_frag(F["xq"], F["xs"], F["wq"], F["ws"], F["y"])
        fb().kv_scale_calibrate(kv["k"], kv["v"], True, kv["ks"], kv["vs"])
        fb().kv_cache_write_fp8(kv["k"], kv["v"], kv["slots"], kv["ks"], kv["vs"], kv["kc"], kv["vc"])

    outs = ([t for L in layers for t in (L["wq"], L["ws"], L["xq"], L["xs"], L["y"])] +
            [kv["ks"], kv["vs"], kv["kc"], kv["vc"], moe["y"], moe["yg"], af["xq"], af["xs"], af["y"]] +
            [t for F in fr for t in (F["wq"], F["ws"], F["xq"], F["xs"], F["y"])])
    announce("graph eager reference")
    work()
    ref = snapshot(outs)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:  # clobber the outputs eagerly between replays
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        announce("graph replay", rep)
        g.replay()
        got = snapshot(outs)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
    # the fragment-order GEMMs give the row-major GEMM's bits, and the
    # fragment-order quantizers its scales
    assert torch.equal(af["y"].view(torch.int16), layers[0]["y"].view(torch.int16))
    for F, L in zip(fr, layers):
        assert torch.equal(F["y"].view(torch.int16), L["y"].view(torch.int16))
        assert torch.equal(F["ws"], L["ws"]) and torch.equal(F["xs"], L["xs"])
