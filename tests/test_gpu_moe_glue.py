"""GPU parity of the MoE expert-FFN glue against the oracle (oracle/moe.py).

Bars: the sort, the gathered codes and scales, the BF16 h and its codes and
scales are bit-exact (index and byte work; h is correctly rounded on both
sides, see silu_mul_quantize_act in the header).  The combine is within one
BF16 rounding plus its float32 accumulation bound (k + 1) * 2^-24 * sum|w y|.
The whole layer (sort -> gather/quantize -> fc1 -> SiLU*up/quantize -> fc2
-> combine) meets the GEMM bar in Frobenius norm and 2^-4 per element (see
layer_case: the chain re-quantizes an intermediate)."""

import numpy as np
import pytest

from helpers import announce, gemm_tolerance_report
from oracle import dequant_act, dequant_weight, quant_act_per_token_group, quant_weight_blockwise
from oracle.bf16 import bf16_bits_to_f64
from oracle.moe import combine, gather_quantize_act, silu_mul_bf16, silu_mul_quantize, sort_by_expert
from synthetic import MOE_QWEN3_30B_A3B, f32_to_bf16_bits, moe_topk

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16(a):
    return f32_to_bf16_bits(np.asarray(a, np.float32))


# ---------------------------------------------------------------- sort
@pytest.mark.parametrize("T,k,E", [(0, 8, 4), (1, 1, 1), (7, 2, 3), (513, 8, 128), (4096, 8, 128), (1000, 4, 300),
                                   (3000, 6, 1), (5000, 8, 64), (20000, 8, 128)])
def test_sort_router_ids(T, k, E):
    announce("moe sort", T, k, E)
    ids, _ = moe_topk(T, E, min(k, E), (90, T)) if T else (np.zeros((0, k), np.int32), None)
    if ids.shape[1] < k:  # fewer experts than slots: repeat ids (duplicates are allowed)
        ids = np.concatenate([ids] * k, axis=1)[:, :k]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    off, rows, pr = fb().moe_sort_by_expert(dev(ids), E)
    roff, rrows, rpr = sort_by_expert(ids, E)
    off, rows, pr = host(off), host(rows), host(pr)
    assert np.array_equal(off, roff)
    assert np.array_equal(rows[:roff[-1]], rrows)
    assert np.array_equal(pr, rpr)


def test_sort_invalid_and_duplicate_ids():
    rng = np.random.default_rng(91)
    for T, k, E in [(5, 3, 4), (1500, 8, 16), (2049, 5, 64)]:
        announce("moe sort invalid", T, k, E)
        ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)
        off, rows, pr = fb().moe_sort_by_expert(dev(ids), E)
        roff, rrows, rpr = sort_by_expert(ids, E)
        assert np.array_equal(host(off), roff)
        assert np.array_equal(host(rows)[:roff[-1]], rrows)
        assert np.array_equal(host(pr), rpr)


# ---------------------------------------------------------------- gather + quantize
@pytest.mark.parametrize("T,k,E,K", [(1, 1, 2, 128), (37, 4, 8, 384), (4096, 8, 128, 2048)])
def test_gather_quantize(T, k, E, K):
    announce("moe gather", T, k, E, K)
    rng = np.random.default_rng([92, T])
    z = rng.normal(0, 1, (T, K)).astype(np.float32)
    z[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 30.0
    x = bf16(z)
    ids, _ = moe_topk(T, E, k, (93, T))
    roff, rrows, _ = sort_by_expert(ids, E)
    rows = np.concatenate([rrows, np.array([-1, T * k + 5], np.int32)])  # two rows naming no token
    q, s = fb().moe_gather_quantize_act(dev(x).view(torch.bfloat16), dev(rows), k)
    q, s = host(q), host(s)
    rq, rs = gather_quantize_act(x, rrows, k)
    assert np.array_equal(q[:len(rrows)], rq) and np.array_equal(s[:len(rrows)], rs)
    assert np.all(q[len(rrows):] == 0) and np.all(s[len(rrows):] == 0)


# ---------------------------------------------------------------- SiLU * up -> BF16 -> 1x128
def silu_case(y, F, label):
    announce("silu_mul", label, y.shape)
    M = y.shape[0]
    h = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    q, s = fb().silu_mul_quantize_act(dev(y).view(torch.bfloat16), h_out=h)
    h, q, s = host(h), host(q), host(s)
    rh = silu_mul_bf16(y, F)
    bad = np.nonzero(h != rh)
    assert bad[0].size == 0, (label, bad[0][:5], bad[1][:5], h[bad][:5], rh[bad][:5])
    rq, rs = silu_mul_quantize(y, F)
    assert np.array_equal(q, rq) and np.array_equal(s, rs), label


@pytest.mark.parametrize("M,F,std", [(1, 8, 1.0), (3, 120, 1.0), (64, 128, 0.5), (257, 768, 1.0), (100, 1000, 3.0),
                                     (2048, 768, 30.0)])
def test_silu_mul_random(M, F, std):
    rng = np.random.default_rng([94, M, F])
    y = bf16(rng.normal(0, std, (M, 2 * F)))
    silu_case(y, F, f"M={M} F={F} std={std}")


def test_silu_mul_ranges_and_specials():
    rng = np.random.default_rng(95)
    F = 256
    rows = []
    # gates beyond the float32 fast range, and tiny / huge products
    rows.append(np.concatenate([rng.uniform(-200, 200, F), rng.normal(0, 1, F)]))
    rows.append(np.concatenate([rng.uniform(-100, -60, F), rng.normal(0, 1e-3, F)]))
    rows.append(np.concatenate([rng.normal(0, 1e-30, F), rng.normal(0, 1e-10, F)]))
    rows.append(np.concatenate([rng.uniform(50, 1e18, F), rng.uniform(-1e18, 1e18, F)]))
    zeros = np.zeros(2 * F)
    zeros[:F:2] = -0.0
    zeros[F + 1::2] = rng.normal(0, 1, F // 2)
    rows.append(zeros)
    y = bf16(np.stack(rows))
    y[4, 1:F:2] = 0x8000  # negative zero gates
    silu_case(y, F, "ranges")


def test_silu_mul_dense_grid_of_gates():
    # every BF16 gate in [-90, 90] against a few up values: exercises the
    # float64 fallback near BF16 midpoints many times
    g = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    gv = bf16_bits_to_f64(g)
    g = g[np.isfinite(gv) & (np.abs(gv) <= 90)]
    F = 1024
    n = (g.size // F) * F
    gates = g[:n].reshape(-1, F)
    for uval in (1.0, -0.7109375, 3.140625):
        y = np.concatenate([gates, np.full(gates.shape, bf16([uval])[0], np.uint16)], axis=1)
        silu_case(y, F, f"gate grid u={uval}")


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("T,k,E,H", [(1, 1, 2, 8), (33, 4, 8, 136), (4096, 8, 128, 2048)])
def test_combine(T, k, E, H):
    announce("moe combine", T, k, E, H)
    rng = np.random.default_rng([96, T])
    ids, w = moe_topk(T, E, k, (97, T))
    _, _, pr = sort_by_expert(ids, E)
    pr = pr.copy()
    pr[::7] = -1  # dropped slots contribute nothing
    M = T * k
    y = bf16(rng.normal(0, 1, (M, H)))
    out = host(fb().moe_combine(dev(y).view(torch.bfloat16), dev(pr), dev(w)))
    ref, mag, _ = combine(y, pr, w)
    got = bf16_bits_to_f64(out)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2.0 ** 16  # BF16 ulp ~ 2^16 f32 ulps
    bound = 0.5 * ulp + (k + 1) * 2.0 ** -24 * mag + 1e-300
    err = np.abs(got - ref)
    assert np.all(err <= bound + 2.0 ** -24 * np.abs(ref)), float(np.max(err / bound))


# ---------------------------------------------------------------- whole layer
def layer_case(T, E, k, H, F, seed, sample=None):
    rng = np.random.default_rng([98, seed])
    x = bf16(rng.standard_normal((T, H), dtype=np.float32))
    w1 = bf16(rng.standard_normal((E, 2 * F, H), dtype=np.float32) * np.float32(0.02))
    w2 = bf16(rng.standard_normal((E, H, F), dtype=np.float32) * np.float32(0.02))
    ids, tw = moe_topk(T, E, k, (99, seed))
    announce("moe layer", T, E, k, H, F)
    w1q, w1s = fb().quantize_weight_blockwise(dev(w1).view(torch.bfloat16))
    w2q, w2s = fb().quantize_weight_blockwise(dev(w2).view(torch.bfloat16))
    out = host(fb().moe_expert_ffn(dev(x).view(torch.bfloat16), dev(ids), dev(tw), w1q, w1s, w2q, w2s))

    # oracle chain, for the sampled tokens only
    toks = np.arange(T) if sample is None else np.sort(rng.choice(T, size=sample, replace=False))
    used = np.unique(ids[toks])  # the oracle quantizes only the experts the sampled tokens use
    w1o = {e: quant_weight_blockwise(w1[e]) for e in used}
    w2o = {e: quant_weight_blockwise(w2[e]) for e in used}
    xq, xs = quant_act_per_token_group(x[toks])
    xd = dequant_act(xq, xs)
    ref = np.zeros((toks.size, H))
    from oracle import round_to_bf16_bits

    for j in range(k):
        ex = ids[toks, j]
        y1 = np.zeros((toks.size, 2 * F))
        for e in np.unique(ex):
            sel = ex == e
            y1[sel] = xd[sel] @ dequant_weight(*w1o[e]).T
        hq, hs = silu_mul_quantize(round_to_bf16_bits(y1), F)
        hd = dequant_act(hq, hs)
        y2 = np.zeros((toks.size, H))
        for e in np.unique(ex):
            sel = ex == e
            y2[sel] = hd[sel] @ dequant_weight(*w2o[e]).T
        ref += tw[toks, j].astype(np.float64)[:, None] * bf16_bits_to_f64(round_to_bf16_bits(y2))
    rep = gemm_tolerance_report(out[toks], ref)
    print("moe layer", T, E, k, H, F, rep, flush=True)
    # The GPU's and the oracle's fc1 outputs are each within the GEMM bar but
    # round to BF16 differently in places (about 1% of them), so a few h
    # codes differ by one E4M3 step (at most 1/8 of |h|).  Each such flip
    # moves one of the F terms of an fc2 output; with F terms of similar
    # size, one term is ~1/sqrt(F) of rms(ref), so a flip moves the output
    # by ~1/(8 sqrt(F)) of it, and an output rarely takes more than a few.
    # The chain keeps the GEMM bar of 1e-2 in Frobenius norm; per element
    # it stays within 1/sqrt(F): 6.25% for F = 256 (this test's small layer
    # measures 3.2%, so it does need more than 1e-2) and 3.6% for the
    # Qwen3-30B-A3B layer's F = 768, which also keeps the 1e-2 bar
    # (measured 0.64% on the full layer).
    assert rep["rel_fro"] <= 1e-2 and rep["rel_max"] <= min(2.0 ** -4, 1.0 / np.sqrt(F)), rep
    return rep


def test_moe_layer_small():
    layer_case(T=96, E=8, k=2, H=256, F=256, seed=1)


def test_moe_layer_qwen3_30b_a3b_sampled():
    c = MOE_QWEN3_30B_A3B
    rep = layer_case(T=c["tokens"], E=c["experts"], k=c["top_k"], H=c["hidden"], F=c["ffn"], seed=2, sample=4)
    assert rep["rel_max"] <= 1e-2, rep


def test_silu_mul_structural_ties():
    # every BF16 gate with |g| < 2^-20 (SiLU(g) u ~ g u / 2) and every gate
    # above 20 (SiLU(g) u ~ g u), against up values with up to 8 significant
    # bits: g u / 2 and g u hit BF16 midpoints exactly, and only the exact
    # side of the midpoint decides the rounding
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(allb)
    fin = np.isfinite(v)
    tiny = allb[fin & (np.abs(v) < 2.0 ** -20)]
    large = allb[fin & (v > 20) & (v < 1e30)]
    rng = np.random.default_rng(97)
    ups = bf16(np.concatenate([[-0.7109375, 3.140625, 1.0078125, -1.9921875], rng.normal(0, 2, 4)]))
    F = 1024
    for name, gates in (("tiny", tiny), ("large", large)):
        n = (gates.size // F) * F
        gg = gates[:n].reshape(-1, F)
        for u in ups:
            y = np.concatenate([gg, np.full(gg.shape, u, np.uint16)], axis=1)
            silu_case(y, F, f"ties {name} u={hex(int(u))}")


def _fused_case(T, k, E, H, F, seed, ids=None, rows=None):
    """fc1 with the SiLU * up quantization in its epilogue against the two
    separate kernels (gathered fc1 GEMM to BF16, then silu_mul_quantize_act):
    the same codes and scales, bit for bit."""
    from synthetic import device_bf16_normal

    announce("fused fc1 SiLU quant", T, k, E, H, F)
    if ids is None:
        ids, _ = moe_topk(T, E, k, (seed, 0))
    off, sp, _ = fb().moe_sort_by_expert(dev(ids.astype(np.int32)), E)
    if rows is not None:
        sp = dev(rows)
    x = device_bf16_normal((T, H), 1.0, seed=seed + 1)
    a, a_s = fb().quantize_act_per_token_group(x)
    w, w_s = fb().quantize_weight_blockwise(device_bf16_normal((E, 2 * F, H), 0.02, seed=seed + 2))
    y1 = fb().grouped_gemm_w8a8_blockscaled_gather(a, a_s, sp, k, w, w_s, off)
    h_ref, hs_ref = fb().silu_mul_quantize_act(y1)
    h, hs = fb().grouped_gemm_w8a8_blockscaled_gather_silu(a, a_s, sp, k, w, w_s, off)
    torch.cuda.synchronize()
    assert torch.equal(h, h_ref), (T, k, E, H, F, int((h != h_ref).sum()))
    assert torch.equal(hs.view(torch.int32), hs_ref.view(torch.int32)), (T, k, E, H, F)


@pytest.mark.parametrize("T,k,E,H,F", [(1, 1, 2, 128, 128), (37, 4, 8, 384, 256), (300, 2, 5, 256, 384),
                                       (513, 8, 16, 1024, 640),
                                       # 10-16 K-blocks, one and several tiles per workgroup
                                       (1, 1, 2, 1280, 128), (37, 4, 8, 1280, 256), (300, 2, 5, 1536, 384),
                                       (700, 8, 6, 2048, 768), (2000, 8, 3, 1408, 256)])
def test_fused_fc1_silu_matches_separate_kernels(T, k, E, H, F):
    _fused_case(T, k, E, H, F, seed=90 + T + H)


def test_fused_fc1_silu_qwen3_30b_a3b():
    """The full Qwen3-30B-A3B fc1 (4096 tokens, top-8 of 128 experts, H = 2048, F = 768)."""
    c = MOE_QWEN3_30B_A3B
    _fused_case(c["tokens"], c["top_k"], c["experts"], c["hidden"], c["ffn"], seed=70)


@pytest.mark.parametrize("H", [256, 2048])
def test_fused_fc1_silu_ragged_and_empty_experts_and_missing_rows(H):
    """Experts with 0, 1, 129 and 300 rows, and gathered rows that name no
    token (negative or past the token count: zero activation rows); with
    2 and 16 K-blocks."""
    T, k, E, F = 250, 2, 6, 256
    counts = [0, 1, 129, 0, 300, 250 * 2 - 430]
    ids = np.repeat(np.arange(E), counts).astype(np.int32)
    ids = np.random.default_rng(3).permutation(ids).reshape(T, k)
    rows = np.random.default_rng(4).integers(-3, T * k + 50, T * k).astype(np.int32)
    _fused_case(T, k, E, H, F, seed=11, ids=ids)
    _fused_case(T, k, E, H, F, seed=12, ids=ids, rows=rows)


def test_fused_fc1_silu_many_float64_decisions_per_lane():
    """fc1 outputs built so that most SiLU*up values sit exactly on a BF16
    midpoint (|gate| < 2^-20, where SiLU(g) u ~ g u / 2 and g u / 2 has nine
    significant bits): the epilogue's float32 path leaves them open, so each
    lane takes many of its 32 values through the float64 decision, one per
    round.  One K-block, one nonzero code per row, so every fc1 output is an
    exact product; the codes and scales must equal the oracle's and the two
    separate kernels', bit for bit."""
    T, k, E, F, K = 300, 1, 2, 128, 128
    announce("fused fc1 SiLU quant, float64 decisions", T, E, F)
    rng = np.random.default_rng(41)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    tok_codes = np.array([0x38, 0x30, 0x40, 0xB8, 0xC8], np.uint8)  # 1, 0.5, 2, -1, -4
    a = np.zeros((T, K), np.uint8)
    a[:, 0] = tok_codes[np.arange(T) % tok_codes.size]
    a_s = np.ones((T, 1), np.float32)
    w = np.zeros((E, 2 * F, K), np.uint8)
    n = np.arange(F)
    # gate rows: powers of two (midpoint products) except every third row (1.375)
    w[:, :F, 0] = np.where(n % 3 == 0, 0x3B, np.array([0x38, 0x30, 0xC0, 0x40])[n % 4])
    w[:, F:, 0] = np.array([0x38, 0xB8, 0x40, 0x30])[n % 4]  # up rows: 1, -1, 2, 0.5
    w_s = np.zeros((E, 2, 1), np.float32)
    w_s[0, :, 0] = [129 * 2.0 ** -37, 1.5]
    w_s[1, :, 0] = [-129 * 2.0 ** -40, 0.75]
    off, sp, _ = fb().moe_sort_by_expert(dev(ids), E)
    h, hs = fb().grouped_gemm_w8a8_blockscaled_gather_silu(dev(a), dev(a_s), sp, k, dev(w), dev(w_s), off)
    y1 = fb().grouped_gemm_w8a8_blockscaled_gather(dev(a), dev(a_s), sp, k, dev(w), dev(w_s), off)
    h_sep, hs_sep = fb().silu_mul_quantize_act(y1)
    # the exact fc1 outputs, in the sorted row order: token sp[m] // k, expert of row m
    offs, rows = host(off).astype(np.int64), host(sp).astype(np.int64)
    expert = np.searchsorted(offs, np.arange(T * k), side="right") - 1
    tok = rows // k
    e4 = {0x38: 1.0, 0x30: 0.5, 0x40: 2.0, 0xB8: -1.0, 0xC8: -4.0, 0x3B: 1.375, 0xC0: -2.0}
    av = np.vectorize(e4.get)(a[tok, 0]).astype(np.float64)
    wv = np.vectorize(e4.get)(w[expert, :, 0]).astype(np.float64)
    scale = np.repeat(w_s[expert, :, 0].astype(np.float64), F, axis=1)
    y = bf16((av[:, None] * wv * scale).astype(np.float32))  # exact in float32
    g = bf16_bits_to_f64(y[:, :F])
    u = bf16_bits_to_f64(y[:, F:])
    half = np.abs(g * u / 2)
    m9 = half / 2.0 ** (np.floor(np.log2(half)) - 8)
    ties = np.mean((m9 == np.round(m9)) & (np.round(m9) % 2 == 1))
    assert ties > 0.5, ties  # most values sit exactly on a midpoint
    rq, rs = silu_mul_quantize(y, F)
    assert np.array_equal(host(h), rq) and np.array_equal(host(hs), rs)
    assert torch.equal(h, h_sep) and torch.equal(hs.view(torch.int32), hs_sep.view(torch.int32))


def test_fused_fc1_silu_shape_errors():
    a = torch.zeros((4, 128), dtype=torch.uint8, device=DEV)
    a_s = torch.ones((4, 1), device=DEV)
    rows = torch.zeros(4, dtype=torch.int32, device=DEV)
    off = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    w = torch.zeros((1, 2 * 192, 128), dtype=torch.uint8, device=DEV)  # F = 192: not a multiple of 128
    with pytest.raises(fb().FP8BQError, match="shape"):
        fb().grouped_gemm_w8a8_blockscaled_gather_silu(a, a_s, rows, 1, w, torch.ones((1, 3, 1), device=DEV), off)


def test_moe_layer_fused_and_separate_are_identical():
    from synthetic import device_bf16_normal

    T, E, k, H, F = 513, 16, 4, 512, 256
    announce("MoE layer fused vs separate", T, E, k, H, F)
    ids, tw = moe_topk(T, E, k, (5, 5))
    x = device_bf16_normal((T, H), 1.0, seed=21)
    w1, w1s = fb().quantize_weight_blockwise(device_bf16_normal((E, 2 * F, H), 0.02, seed=22))
    w2, w2s = fb().quantize_weight_blockwise(device_bf16_normal((E, H, F), 0.02, seed=23))
    y0 = fb().moe_expert_ffn(x, dev(ids), dev(tw), w1, w1s, w2, w2s, fused=False)
    y1 = fb().moe_expert_ffn(x, dev(ids), dev(tw), w1, w1s, w2, w2s, fused=True)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_grouped_gemm_k_zero_gives_zeros():
    """K = 0 experts: the zero products are stored (plain and gathered)."""
    m, n, g = 40, 256, 3
    off = torch.tensor([0, 10, 10, 40], dtype=torch.int32, device=DEV)
    a = torch.empty((m, 0), dtype=torch.uint8, device=DEV)
    a_s = torch.empty((m, 0), dtype=torch.float32, device=DEV)
    w = torch.empty((g, n, 0), dtype=torch.uint8, device=DEV)
    w_s = torch.empty((g, 2, 0), dtype=torch.float32, device=DEV)
    y = torch.full((m, n), 1.0, dtype=torch.bfloat16, device=DEV)
    fb().grouped_gemm_w8a8_blockscaled(a, a_s, w, w_s, off, y)
    assert torch.count_nonzero(y.float()) == 0
    y.fill_(1.0)
    rows = torch.arange(m, dtype=torch.int32, device=DEV)
    fb().grouped_gemm_w8a8_blockscaled_gather(a, a_s, rows, 1, w, w_s, off, y)
    assert torch.count_nonzero(y.float()) == 0
