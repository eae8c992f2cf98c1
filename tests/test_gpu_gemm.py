"""GPU parity of the block-scaled GEMM and the grouped (MoE) GEMM.

Acceptance per GEMM (and per expert): relative Frobenius error and worst
element error (against max(|y_ref|, rms(y_ref))) both <= 1e-2 versus the
float64 oracle, plus >= 90% of outputs equal to the oracle's own BF16
rounding (FP32 accumulation changes only last-bit ties).

Inputs to the GEMM-only cases are quantized by the oracle on the host and
uploaded; the full-size cases run the whole GPU path (quantizers, then
GEMM) and compare sampled outputs with the oracle's quantize-then-multiply
of the same BF16 inputs.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from helpers import (
    ROOT,
    announce,
    assert_gemm_close,
    bf16_bits_to_device,
    device_to_bits,
    sample_cols,
    sampled_gemm_ref,
)
from synthetic import LAYER_SHAPES_QWEN3_8B, MOE_QWEN3_30B_A3B, activations, bf16_normal, gather_rows, moe_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_gemm(fb, qa, sa, qw, sw, tile=None):
    y = fb.gemm_w8a8_blockscaled(_dev(qa), _dev(sa), _dev(qw), _dev(sw), tile=tile)
    return device_to_bits(y)


def _oracle_inputs(m, n, k, seed, n_out=0, mult=1.0):
    x, _ = activations(m, k, (seed, 0), n_outliers=n_out, outlier_mult=mult)
    w = bf16_normal((n, k), 0.02, (seed, 1))
    qa, sa = oracle.quant_act_per_token_group(x)
    qw, sw = oracle.quant_weight_blockwise(w)
    return qa, sa, qw, sw


def test_gemm_tiny_config(fb):
    announce("gemm tiny 32x384x512")
    qa, sa, qw, sw = _oracle_inputs(32, 384, 512, 30, 4, 50.0)
    rep = assert_gemm_close(gpu_gemm(fb, qa, sa, qw, sw), oracle.gemm_ref(qa, sa, qw, sw))
    print(rep)


@pytest.mark.parametrize("m,n,k", [(100, 200, 256), (1, 1, 128), (130, 129, 384), (257, 130, 1024), (3, 1000, 128),
                                   (64, 128, 2048)])
def test_gemm_ragged(fb, m, n, k):
    announce("gemm ragged", m, n, k)
    qa, sa, qw, sw = _oracle_inputs(m, n, k, 31 + m)
    assert_gemm_close(gpu_gemm(fb, qa, sa, qw, sw), oracle.gemm_ref(qa, sa, qw, sw))


TILES = ["skinny64", "skinny48", "skinny96", "wide", "decode_panel", "deep", "panel192"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (37, 130, 256), (130, 300, 384), (257, 129, 1024), (300, 520, 2048)])
def test_gemm_every_tile_kernel(fb, tile, m, n, k):
    """Each tile kernel on ragged shapes and 1..16 K-blocks (odd and even
    trip counts of the pipelined loops), named through gemm_w8a8_blockscaled_tile."""
    announce("gemm tile", tile, m, n, k)
    qa, sa, qw, sw = _oracle_inputs(m, n, k, 90 + m + n)
    assert_gemm_close(gpu_gemm(fb, qa, sa, qw, sw, tile), oracle.gemm_ref(qa, sa, qw, sw))


PANEL_TILES = ["wide", "decode_panel", "deep", "panel192"]


@pytest.mark.parametrize("m", [100, 128, 150, 200, 257])
def test_gemm_panel_tiles_same_bits(fb, m):
    """The panel tiles accumulate every output over the K-blocks in K order
    with the same per-K-block scale FMA, so they give the same bits whatever
    their shape, their number of stages, and which waves issue the loads.
    The row counts put ragged last tiles with empty rows of waves, whose
    waves 4-7 take the loads, into each panel: 100 and 128 rows (the 128 x
    256 panel's split form; the 256-row panels' last row of waves empty),
    150 (the 256 x 256 tile with one row of waves empty), 200 and 257 (the
    192 x 128 panel's last tile of 72 or 1 rows), beside full tiles."""
    announce("gemm panel tiles same bits", m)
    qa, sa, qw, sw = _oracle_inputs(m, 520, 1024, 60 + m)
    ys = {tile: gpu_gemm(fb, qa, sa, qw, sw, tile) for tile in PANEL_TILES}
    assert_gemm_close(ys["wide"], oracle.gemm_ref(qa, sa, qw, sw))
    for tile in PANEL_TILES[1:]:
        assert np.array_equal(ys[tile], ys["wide"]), tile


@pytest.mark.parametrize("tile", TILES)
def test_gemm_every_tile_random_scales(fb, tile):
    """Each tile kernel with a different scale in every weight block,
    activation row and K-block (tiles that straddle scale blocks, a partial
    last block, zero-scale rows).  The spread (2^-3..2^3) keeps every
    K-block's term visible in the sum, and each (row, 128-column block)
    is checked on its own, so a scale applied to the wrong rows, block or
    K-block fails."""
    announce("gemm tile random scales", tile)
    rng = np.random.default_rng(35)
    m, n, k = 300, 520, 640
    qa = rng.integers(0, 256, (m, k)).astype(np.uint8)
    qw = rng.integers(0, 256, (n, k)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    qw[(qw & 0x7F) == 0x7F] = 0x80
    sa = np.exp2(rng.uniform(-3, 3, (m, k // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(-3, 3, ((n + 127) // 128, k // 128))).astype(np.float32)
    zero_rows = [0, 63, 64, 257]
    sa[zero_rows] = 0
    y = gpu_gemm(fb, qa, sa, qw, sw, tile)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    assert np.all((y[zero_rows] & 0x7FFF) == 0)
    for r in range(m):
        if r in zero_rows:
            continue
        for c0 in range(0, n, 128):
            assert_gemm_close(y[r:r + 1, c0:c0 + 128], ref[r:r + 1, c0:c0 + 128], min_exact=0.5)


def test_gemm_k_zero_gives_zeros(fb):
    announce("gemm K = 0")
    y = fb.gemm_w8a8_blockscaled(torch.empty((5, 0), dtype=torch.uint8, device="cuda"),
                                 torch.empty((5, 0), dtype=torch.float32, device="cuda"),
                                 torch.empty((7, 0), dtype=torch.uint8, device="cuda"),
                                 torch.empty((1, 0), dtype=torch.float32, device="cuda"))
    assert torch.count_nonzero(y.float()) == 0 and y.shape == (5, 7)


def test_gemm_random_codes_and_scales(fb):
    """All finite codes, scales spread over 2^-40..2^40, zero-scale rows."""
    announce("gemm random codes 192x256x640")
    rng = np.random.default_rng(32)
    m, n, k = 192, 256, 640
    qa = rng.integers(0, 256, (m, k)).astype(np.uint8)
    qw = rng.integers(0, 256, (n, k)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    qw[(qw & 0x7F) == 0x7F] = 0x80
    sa = np.exp2(rng.uniform(-40, 40, (m, k // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(-40, 40, (2, k // 128))).astype(np.float32)
    sa[5] = 0
    y = gpu_gemm(fb, qa, sa, qw, sw)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    # per-row relative check: row magnitudes differ by up to 2^80
    for r in range(m):
        if not np.any(ref[r]):
            assert np.all((y[r] & 0x7FFF) == 0)
            continue
        assert_gemm_close(y[r:r + 1], ref[r:r + 1], min_exact=0.5)


def test_gemm_one_hot_rows(fb):
    announce("gemm one-hot rows")
    rng = np.random.default_rng(33)
    n, k = 256, 384
    w = bf16_normal((n, k), 0.02, (33, 0))
    qw, sw = oracle.quant_weight_blockwise(w)
    cols = np.array([0, 127, 128, 255, 300, 383])
    qa = np.zeros((len(cols), k), np.uint8)
    qa[np.arange(len(cols)), cols] = 0x38
    sa = np.ones((len(cols), 3), np.float32)
    y = gpu_gemm(fb, qa, sa, qw, sw)
    want = oracle.round_to_bf16_bits(oracle.dequant_weight(qw, sw)[:, cols].T)
    assert np.array_equal(y, want)  # a single exact product: bit-exact
    _ = rng


@pytest.mark.parametrize("n,k", [(1024, 4096), (512, 12288)])
def test_gemm_decode_shaped_full(fb, n, k):
    announce("gemm decode-shaped full 256 x", n, k)
    qa, sa, qw, sw = _oracle_inputs(256, n, k, 34)
    assert_gemm_close(gpu_gemm(fb, qa, sa, qw, sw), oracle.gemm_ref(qa, sa, qw, sw))


def _full_path(fb, x_bits, w_bits):
    xq, xs = fb.quantize_act_per_token_group(bf16_bits_to_device(x_bits))
    wq, ws = fb.quantize_weight_blockwise(bf16_bits_to_device(w_bits))
    return fb.gemm_w8a8_blockscaled(xq, xs, wq, ws)


@pytest.mark.parametrize("idx", range(len(LAYER_SHAPES_QWEN3_8B)))
@pytest.mark.parametrize("m", [256, 8192])
def test_full_path_qwen3_8b_sampled(fb, idx, m):
    name, n, k = LAYER_SHAPES_QWEN3_8B[idx]
    announce("full path qwen3-8b", name, m, n, k)
    n_out = round(0.01 * k) if m == 8192 else 0
    x, _ = activations(m, k, (40 + idx, m), n_outliers=n_out, outlier_mult=30.0)
    w = bf16_normal((n, k), 0.02, (41, idx))
    y = _full_path(fb, x, w)
    rng = np.random.default_rng(idx * 7 + m)
    rows = np.sort(rng.choice(m, 64, replace=False))
    cols = sample_cols(rng, n)
    ref = sampled_gemm_ref(x[rows], w, cols)
    got = device_to_bits(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].contiguous())
    assert_gemm_close(got, ref)


# ------------------------------------------------------------ grouped GEMM

def _grouped_oracle_inputs(counts, n, k, seed):
    g = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m = int(off[-1])
    x, _ = activations(max(m, 1), k, (seed, 0))
    x = x[:m]
    w = bf16_normal((g, n, k), 0.02, (seed, 1))
    qa, sa = oracle.quant_act_per_token_group(x)
    qw, sw = oracle.quant_weight_blockwise(w)
    return qa, sa, qw, sw, off


def gpu_grouped(fb, qa, sa, qw, sw, off, tile=None):
    y = fb.grouped_gemm_w8a8_blockscaled(_dev(qa), _dev(sa), _dev(qw), _dev(sw), _dev(off), tile=tile)
    return device_to_bits(y)


@pytest.mark.parametrize("tile", ["wide", "decode_panel", "deep", "deep_persistent"])
@pytest.mark.parametrize("counts", [[3, 0, 17, 1, 0], [0, 0, 300, 0], [129], [0, 128, 0, 1, 255, 0, 0, 2],
                                    [1] * 40, [257, 511, 70]])
def test_grouped_small(fb, tile, counts):
    announce("grouped small", tile, counts)
    qa, sa, qw, sw, off = _grouped_oracle_inputs(counts, 256, 384, 50 + len(counts))
    y = gpu_grouped(fb, qa, sa, qw, sw, off, tile)
    ref = oracle.grouped_gemm_ref(qa, sa, qw, sw, off)
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert_gemm_close(y[lo:hi], ref[lo:hi])


@pytest.mark.parametrize("tile", ["wide", "decode_panel", "deep", "deep_persistent"])
@pytest.mark.parametrize("counts,div", [([3, 0, 17, 1, 0], 1), ([0, 128, 0, 1, 255, 0, 0, 2], 8), ([257, 511, 70], 3),
                                        ([1] * 40, 2)])
def test_grouped_gather(fb, tile, counts, div):
    """Row m of the output uses row a_rows[m] // div of a (MoE tokens read
    through their routed pairs); rows naming no row of a give zeros."""
    announce("grouped gather", tile, counts, div)
    n, k = 256, 384
    g = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m = int(off[-1])
    m_a = max(7, m // 3)
    x, _ = activations(m_a, k, (70 + g, 0))
    w = bf16_normal((g, n, k), 0.02, (70 + g, 1))
    qa, sa = oracle.quant_act_per_token_group(x)
    qw, sw = oracle.quant_weight_blockwise(w)
    rng = np.random.default_rng(71 + g)
    rows = rng.integers(0, m_a * div, size=m).astype(np.int32)
    if m > 4:
        rows[1] = -5               # no row
        rows[m // 2] = m_a * div   # one past the last row
    y = device_to_bits(fb.grouped_gemm_w8a8_blockscaled_gather(_dev(qa), _dev(sa), _dev(rows), div, _dev(qw),
                                                                _dev(sw), _dev(off), tile=tile))
    src = rows // div
    valid = (rows >= 0) & (src < m_a)
    qg = np.where(valid[:, None], qa[np.clip(src, 0, m_a - 1)], 0).astype(np.uint8)
    sg = np.where(valid[:, None], sa[np.clip(src, 0, m_a - 1)], 0).astype(np.float32)
    ref = oracle.grouped_gemm_ref(qg, sg, qw, sw, off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert_gemm_close(y[lo:hi], ref[lo:hi])
    assert np.all(y[~valid] == 0)


def test_grouped_single_group_equals_dense(fb):
    announce("grouped G=1 vs dense")
    qa, sa, qw, sw, off = _grouped_oracle_inputs([200], 384, 512, 60)
    yg = gpu_grouped(fb, qa, sa, qw, sw, off)
    yd = gpu_gemm(fb, qa, sa, qw[0], sw[0])
    ref = oracle.gemm_ref(qa, sa, qw[0], sw[0])
    assert_gemm_close(yg, ref)
    assert_gemm_close(yd, ref)
    # the two launches may use different tilings (summation orders): they
    # agree except for last-bit rounding of a few outputs
    assert np.mean(yg == yd) >= 0.95


def test_grouped_ragged_n(fb):
    announce("grouped ragged N=200")
    qa, sa, qw, sw, off = _grouped_oracle_inputs([5, 130, 0, 7], 200, 256, 61)
    y = gpu_grouped(fb, qa, sa, qw, sw, off)
    ref = oracle.grouped_gemm_ref(qa, sa, qw, sw, off)
    assert_gemm_close(y, ref)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_moe_full_size_sampled(fb, proj):
    """Qwen3-30B-A3B expert layer at full size: GPU quantizers + grouped GEMM."""
    cfg = MOE_QWEN3_30B_A3B
    g, t = cfg["experts"], cfg["tokens"]
    n, k = cfg[proj]
    announce("grouped moe full", proj, g, n, k)
    tok, exp, off = moe_routing(t, g, cfg["top_k"], (70, 0))
    m = int(off[-1])
    if proj == "gate_up":
        h, _ = activations(t, k, (70, 1))
        x = gather_rows(h, tok)
    else:
        x, _ = activations(m, k, (70, 2))
    w = bf16_normal((g, n, k), 0.02, (70, 3 if proj == "gate_up" else 4))
    xq, xs = fb.quantize_act_per_token_group(bf16_bits_to_device(x))
    wq, ws = fb.quantize_weight_blockwise(bf16_bits_to_device(w))
    y = fb.grouped_gemm_w8a8_blockscaled(xq, xs, wq, ws, _dev(off))
    rng = np.random.default_rng(71)
    for e in rng.choice(g, 6, replace=False):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.sort(rng.choice(np.arange(lo, hi), min(16, hi - lo), replace=False))
        cols = sample_cols(rng, n, blocks=2, per_block=16)
        ref = sampled_gemm_ref(x[rows], w[e], cols)
        got = device_to_bits(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].contiguous())
        assert_gemm_close(got, ref)


def test_offsets_check(fb):
    """The offsets checker rejects offsets that break the contract; valid
    offsets pass and the GEMM runs as usual."""
    announce("offsets check")
    qa, sa, qw, sw, off = _grouped_oracle_inputs([5, 0, 9], 128, 256, 80)
    fb.check_group_offsets(_dev(off), 14)
    y = gpu_grouped(fb, qa, sa, qw, sw, off)
    assert_gemm_close(y, oracle.grouped_gemm_ref(qa, sa, qw, sw, off))
    for bad in ([0, 9, 5, 14], [1, 5, 5, 14], [0, 5, 5, 13]):
        with pytest.raises(fb.FP8BQError, match="invalid shape"):
            fb.check_group_offsets(_dev(np.array(bad, np.int32)), 14)


_DEBUG_MODE_CHILD = """
import numpy as np, torch
import fp8_blockwise_quantized_quantize_amd as fb
a = torch.zeros((14, 256), dtype=torch.uint8, device="cuda")
sa = torch.ones((14, 2), device="cuda")
w = torch.zeros((3, 128, 256), dtype=torch.uint8, device="cuda")
sw = torch.ones((3, 1, 2), device="cuda")
rows = torch.arange(14, dtype=torch.int32, device="cuda")
good = torch.tensor([0, 5, 5, 14], dtype=torch.int32, device="cuda")
fb.grouped_gemm_w8a8_blockscaled(a, sa, w, sw, good)
for bad in ([0, 9, 5, 14], [1, 5, 5, 14], [0, 5, 5, 13]):
    off = torch.tensor(bad, dtype=torch.int32, device="cuda")
    for call in (lambda: fb.grouped_gemm_w8a8_blockscaled(a, sa, w, sw, off),
                 lambda: fb.grouped_gemm_w8a8_blockscaled_gather(a, sa, rows, 1, w, sw, off)):
        try:
            call()
        except fb.FP8BQError as e:
            assert "invalid shape" in str(e)
        else:
            raise SystemExit("bad offsets accepted")
torch.cuda.synchronize()
print("debug mode ok", flush=True)
"""


def test_offsets_debug_mode_from_the_environment():
    """FP8BQ_CHECK_OFFSETS=1 (read once per process, so in a process of its
    own) makes every grouped call check its offsets and reject broken ones
    before launching anything."""
    import subprocess
    import sys

    announce("offsets debug mode (child process)")
    env = dict(os.environ, FP8BQ_CHECK_OFFSETS="1")
    r = subprocess.run([sys.executable, "-c", _DEBUG_MODE_CHILD], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "debug mode ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.parametrize("tile", TILES)
def test_gemm_largest_k(fb, tile):
    """K = 2^22, the largest K the boundary accepts: a 256-row activation
    panel then spans 2^30 bytes, still addressed with 32-bit buffer offsets
    (the 256-row tiles read rows up to 255 * 2^22 bytes in), over 32768
    K-blocks.  Random E4M3 codes (NaN codes replaced by zero) and random
    scales, drawn on the GPU; rows 0, 1, 128 and 255 are checked against the
    oracle on the host.  One K-block more is rejected before anything runs."""
    k = 1 << 22
    m, n = 256, 3
    announce("gemm largest K", tile, m, n, k)
    g = torch.Generator(device="cuda").manual_seed(2201)
    qa = torch.randint(0, 256, (m, k), generator=g, dtype=torch.uint8, device="cuda")
    qa[(qa & 0x7F) == 0x7F] = 0
    qw = torch.randint(0, 256, (n, k), generator=g, dtype=torch.uint8, device="cuda")
    qw[(qw & 0x7F) == 0x7F] = 0
    sa = torch.rand((m, k // 128), generator=g, device="cuda") + 0.5
    sw = torch.rand((1, k // 128), generator=g, device="cuda") + 0.5
    y = fb.gemm_w8a8_blockscaled(qa, sa, qw, sw, tile=tile)
    torch.cuda.synchronize()
    rows = [0, 1, 128, 255]
    ref = oracle.gemm_ref(qa[rows].cpu().numpy(), sa[rows].cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy())
    got = device_to_bits(y)[rows]
    print(assert_gemm_close(got, ref))
    del qa, y
    over = k + 128
    a1 = torch.zeros((1, over), dtype=torch.uint8, device="cuda")
    s1 = torch.ones((1, over // 128), device="cuda")
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.gemm_w8a8_blockscaled(a1, s1, a1, s1)


@pytest.mark.parametrize("tile", [None, "deep_persistent"])
def test_grouped_more_experts_than_the_persistent_table(fb, tile):
    """1100 experts, most of them empty: above the 1024 experts whose tile
    prefix the persistent kernel keeps in LDS, so the default (and even a
    forced deep_persistent) runs the per-tile kernel; 1024 experts exactly
    still run persistent."""
    for g_total in (1100, 1024):
        announce("grouped many experts", tile, g_total)
        rng = np.random.default_rng(g_total)
        counts = np.zeros(g_total, np.int64)
        busy = rng.choice(g_total, 24, replace=False)
        counts[busy] = rng.integers(1, 300, 24)
        counts[-1] = 5  # the last expert's rows end the offsets
        qa, sa, qw, sw, off = _grouped_oracle_inputs(counts, 128, 256, 90 + g_total)
        y = gpu_grouped(fb, qa, sa, qw, sw, off, tile)
        ref = oracle.grouped_gemm_ref(qa, sa, qw, sw, off)
        for e in np.nonzero(counts)[0]:
            lo, hi = off[e], off[e + 1]
            assert_gemm_close(y[lo:hi], ref[lo:hi])


# ---------------------------------------------------------------- K split

@pytest.mark.parametrize("m,n,k", [(16, 4096, 12288), (128, 4096, 12288), (64, 1000, 8192), (100, 300, 16384),
                                   (65, 129, 8192), (33, 520, 9344), (1, 256, 8192)])
def test_gemm_splitk_against_oracle(fb, m, n, k):
    """The K-split GEMM for few activation rows and long K: the Qwen3-8B
    down projection (K = 12288) at 16 and 128 tokens, and ragged shapes
    (partial tiles in M and N, a K-block count the pieces divide unevenly,
    one row) meet the 1e-2 bar against the oracle; the workspace the size
    query names is used, a smaller one is refused, and two calls with
    different workspace contents give the same bits (a fixed summation
    order)."""
    announce("gemm split-K", m, n, k)
    qa, sa, qw, sw = _oracle_inputs(m, n, k, 140 + m + n, 4, 30.0)
    need = fb.splitk_workspace_bytes(m, n, k)
    assert need > 0 and need % (4 * m * n) == 0 and 2 <= need // (4 * m * n) <= 8
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    y = fb.gemm_w8a8_blockscaled_splitk(_dev(qa), _dev(sa), _dev(qw), _dev(sw), workspace=ws)
    got = device_to_bits(y)
    print(assert_gemm_close(got, oracle.gemm_ref(qa, sa, qw, sw)))
    ws.fill_(0xFF)
    y2 = fb.gemm_w8a8_blockscaled_splitk(_dev(qa), _dev(sa), _dev(qw), _dev(sw), workspace=ws)
    assert np.array_equal(device_to_bits(y2), got)
    with pytest.raises(fb.FP8BQError, match="workspace"):
        fb.gemm_w8a8_blockscaled_splitk(_dev(qa), _dev(sa), _dev(qw), _dev(sw), workspace=ws[: need - 16])


@pytest.mark.parametrize("m,n,k", [(16, 4096, 4096), (256, 4096, 12288), (128, 4096, 8192), (512, 4096, 65536),
                                   (64, 24576, 8192), (256, 6144, 4096)])
def test_gemm_splitk_unsplit_shapes_run_the_plain_gemm(fb, m, n, k):
    """Shapes the split rule leaves whole (pieces of fewer than 8 K-blocks,
    M too large against K, M > 256, weight tiles that fill the CUs; the
    Qwen3-8B decode shapes at M = 256) need no workspace and give the plain
    GEMM's bits."""
    announce("gemm split-K unsplit", m, n, k)
    assert fb.splitk_workspace_bytes(m, n, k) == 0
    g = torch.Generator(device="cuda").manual_seed(m + n + k)
    qa = torch.randint(0, 256, (m, k), generator=g, dtype=torch.uint8, device="cuda")
    qa[(qa & 0x7F) == 0x7F] = 0
    qw = torch.randint(0, 256, (n, k), generator=g, dtype=torch.uint8, device="cuda")
    qw[(qw & 0x7F) == 0x7F] = 0
    sa = torch.rand((m, k // 128), generator=g, device="cuda") + 0.5
    sw = torch.rand(((n + 127) // 128, k // 128), generator=g, device="cuda") + 0.5
    y0 = fb.gemm_w8a8_blockscaled(qa, sa, qw, sw)
    y1 = fb.gemm_w8a8_blockscaled_splitk(qa, sa, qw, sw, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
