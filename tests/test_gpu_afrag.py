"""GPU parity of the fragment-order activation path: the quantizer writing
the codes in MFMA fragment order, and the GEMM that reads them.

The quantizer must give the oracle's codes, permuted by the oracle's
fragment order, and the oracle's scales, bit for bit.  The GEMM must meet
the GEMM bar against the exact oracle and give the same bits as the
row-major GEMM with the tile the cost model picks for the shape (same
per-element arithmetic and order).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import announce, assert_gemm_close, bf16_bits_to_device, device_to_bits
from synthetic import LAYER_SHAPES_QWEN3_8B, activations, bf16_normal, device_bf16_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


@pytest.mark.parametrize("m,k", [(16, 128), (48, 384), (272, 2048), (256, 12288)])
def test_quantizer_fragment_order(fb, m, k):
    announce("afrag quant", m, k)
    x, _ = activations(m, k, (m, k), n_outliers=max(1, k // 100), outlier_mult=30.0)
    q, s = fb.quantize_act_per_token_group_frag(bf16_bits_to_device(x))
    oq, os_ = oracle.quant_act_per_token_group(x)
    assert np.array_equal(q.cpu().numpy(), oracle.act_fragment_order(oq))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("m,k", [(8192, 4096), (4112, 2176), (8208, 2176)])
def test_quantizer_fragment_order_matches_row_major_prefill(fb, m, k):
    """At the prefill size, and at odd unit counts with a ragged last
    workgroup (4369 and 8721 units of 16 rows x 128): the fragment codes are
    the row-major GPU codes permuted (the row-major quantizer is itself
    checked against the oracle)."""
    announce("afrag quant prefill", m, k)
    x = device_bf16_normal((m, k), 1.0, seed=9)
    q, s = fb.quantize_act_per_token_group(x)
    qf, sf = fb.quantize_act_per_token_group_frag(x)
    perm = q.view(m // 16, 16, k // 128, 2, 4, 16).permute(0, 2, 3, 4, 1, 5).contiguous().view(m, k)
    assert torch.equal(qf, perm) and torch.equal(sf, s)


def test_quantizer_frag_multi_matches_oracle(fb):
    """One launch over the four decode activations of a Qwen3-8B layer
    (M = 256) plus small and empty ones: each gets the oracle's codes in
    fragment order and the oracle's scales."""
    shapes = [(256, 4096), (256, 4096), (256, 4096), (256, 12288), (16, 128), (48, 384), (0, 256), (272, 2048)]
    announce("afrag quant multi", shapes)
    xs_bits = [activations(m, k, (m, k, i), n_outliers=max(1, k // 100), outlier_mult=30.0)[0] if m else
               np.zeros((m, k), np.uint16) for i, (m, k) in enumerate(shapes)]
    res = fb.quantize_acts_per_token_group_frag_multi([bf16_bits_to_device(b) for b in xs_bits])
    torch.cuda.synchronize()
    for (q, s), b, (m, k) in zip(res, xs_bits, shapes):
        if m == 0:
            continue
        oq, os_ = oracle.quant_act_per_token_group(b)
        assert np.array_equal(q.cpu().numpy(), oracle.act_fragment_order(oq)), (m, k)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), (m, k)


@pytest.mark.parametrize("m,k", [(24, 256), (16, 200)])
def test_quantizer_frag_multi_shape_errors(fb, m, k):
    ok = torch.zeros((16, 128), dtype=torch.bfloat16, device="cuda")
    bad = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.quantize_acts_per_token_group_frag_multi([ok, bad])


@pytest.mark.parametrize("m,n,k", [(16, 130, 256), (48, 384, 768), (272, 520, 512), (272, 528, 512),
                                   (256, 256, 2048), (80, 20480, 256), (208, 24576, 256),
                                   (32, 256, 384), (512, 512, 640), (144, 24576, 128), (208, 24576, 384),
                                   (80, 20480, 384), (256, 6128, 512), (64, 24560, 384), (208, 6144, 640)])
def test_gemm_afrag_against_oracle_and_row_major(fb, m, n, k):
    """Every tile form: 64-, 48- and 96-row K-split tiles, the 256 x 256
    panel, the 128 x 256 decode panel (M = 80: one ragged tile of activation
    rows) and the 192 x 128 panel (M = 208: a second, ragged row tile).
    N = 6128 and 24560 put an 80-row last tile on the 96-row skinny tile (the
    row-major form runs the 48-row one there: the same bits), M = 208 a
    ragged row tile on it.  Where N % 16 == 0 the same product with the
    weights in fragment order too (N = 528: a ragged last weight scale block
    of 16 rows).  K = 128, 384 and 640: odd numbers of K-blocks on every tile
    form."""
    announce("afrag gemm", m, n, k)
    x, _ = activations(m, k, (m, n, k, 0))
    w = bf16_normal((n, k), 0.02, (m, n, k, 1))
    qa, sa = oracle.quant_act_per_token_group(x)
    qw, sw = oracle.quant_weight_blockwise(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = fb.gemm_w8a8_blockscaled_afrag(dev(oracle.act_fragment_order(qa)), dev(sa), dev(qw), dev(sw))
    got = device_to_bits(y)
    assert_gemm_close(got, oracle.gemm_ref(qa, sa, qw, sw))
    ref = device_to_bits(fb.gemm_w8a8_blockscaled(dev(qa), dev(sa), dev(qw), dev(sw)))
    assert np.array_equal(got, ref)
    if n % 16 == 0:
        yf = fb.gemm_w8a8_blockscaled_frag(dev(oracle.act_fragment_order(qa)), dev(sa),
                                           dev(oracle.act_fragment_order(qw)), dev(sw))
        assert np.array_equal(device_to_bits(yf), ref)


@pytest.mark.parametrize("m", [256, 208, 144, 128, 64, 48, 16])
def test_gemm_afrag_decode_shapes_bit_identical(fb, m):
    """The Qwen3-8B layer shapes at decode batch sizes: the fragment-order
    GEMM picks the row-major GEMM's tile in its fragment-order form (K split
    over the waves of a 64- or 48-row tile, or a panel) and gives its bits."""
    for _, n, k in LAYER_SHAPES_QWEN3_8B:
        announce("afrag gemm decode", m, n, k)
        x = device_bf16_normal((m, k), 1.0, seed=13)
        wb = device_bf16_normal((n, k), 0.02, seed=14)
        wq, ws = fb.quantize_weight_blockwise(wb)
        wqf, _ = fb.quantize_weight_blockwise_frag(wb)
        q, s = fb.quantize_act_per_token_group(x)
        qf, _ = fb.quantize_act_per_token_group_frag(x)
        y0 = fb.gemm_w8a8_blockscaled(q, s, wq, ws)
        y1 = fb.gemm_w8a8_blockscaled_afrag(qf, s, wq, ws)
        y2 = fb.gemm_w8a8_blockscaled_frag(qf, s, wqf, ws)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), (m, n, k)
        assert torch.equal(y0.view(torch.int16), y2.view(torch.int16)), (m, n, k)


@pytest.mark.parametrize("n,k", [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (2048, 384), (2048, 640)])
def test_gemm_afrag_prefill_bit_identical(fb, n, k):
    """The four Qwen3-8B prefill shapes (M = 8192), and the 256 x 256 panel on
    odd numbers of K-blocks: same bits as the row-major tile."""
    m = 8192
    announce("afrag gemm prefill", m, n, k)
    x = device_bf16_normal((m, k), 1.0, seed=11)
    wb = device_bf16_normal((n, k), 0.02, seed=12)
    wq, ws = fb.quantize_weight_blockwise(wb)
    wqf, _ = fb.quantize_weight_blockwise_frag(wb)
    q, s = fb.quantize_act_per_token_group(x)
    qf, _ = fb.quantize_act_per_token_group_frag(x)
    y0 = fb.gemm_w8a8_blockscaled(q, s, wq, ws, tile="wide")
    y1 = fb.gemm_w8a8_blockscaled_afrag(qf, s, wq, ws)
    y2 = fb.gemm_w8a8_blockscaled_frag(qf, s, wqf, ws)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


def test_gemm_afrag_largest_k(fb):
    """K = 2^22: 256 rows of fragment-order codes span 2^30 bytes (with the
    16 weight rows in fragment order too)."""
    m, n, k = 256, 16, 1 << 22
    announce("afrag gemm largest K", m, n, k)
    g = torch.Generator(device="cuda").manual_seed(2202)
    qa = torch.randint(0, 256, (m, k), generator=g, dtype=torch.uint8, device="cuda")
    qa[(qa & 0x7F) == 0x7F] = 0
    qw = torch.randint(0, 256, (n, k), generator=g, dtype=torch.uint8, device="cuda")
    qw[(qw & 0x7F) == 0x7F] = 0
    sa = torch.rand((m, k // 128), generator=g, device="cuda") + 0.5
    sw = torch.rand((1, k // 128), generator=g, device="cuda") + 0.5
    qf = qa.view(m // 16, 16, k // 128, 2, 4, 16).permute(0, 2, 3, 4, 1, 5).contiguous().view(m, k)
    y0 = fb.gemm_w8a8_blockscaled(qa, sa, qw, sw)
    del qa
    y1 = fb.gemm_w8a8_blockscaled_afrag(qf, sa, qw, sw)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    qwf = qw.view(n // 16, 16, k // 128, 2, 4, 16).permute(0, 2, 3, 4, 1, 5).contiguous().view(n, k)
    y2 = fb.gemm_w8a8_blockscaled_frag(qf, sa, qwf, sw)
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("shape", [(128, 128), (384, 512), (16, 256), (144, 384), (2, 144, 256)])
def test_weight_quantizer_fragment_order(fb, shape):
    """The oracle's codes permuted into fragment order and the oracle's
    scales; (144, 384): a last block of 16 rows (element-wise path);
    (2, 144, 256): the batched form."""
    announce("frag weight quant", shape)
    bits = bf16_normal(shape, 0.02, (len(shape),) + shape)
    q, s = fb.quantize_weight_blockwise_frag(bf16_bits_to_device(bits))
    mats = bits if len(shape) == 3 else bits[None]
    for b in range(mats.shape[0]):
        oq, os_ = oracle.quant_weight_blockwise(mats[b])
        gq = q.cpu().numpy() if len(shape) == 2 else q[b].cpu().numpy()
        gs = s.cpu().numpy() if len(shape) == 2 else s[b].cpu().numpy()
        assert np.array_equal(gq, oracle.act_fragment_order(oq)), (shape, b)
        assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), (shape, b)


def test_weight_quantizer_fragment_order_multi(fb):
    """One launch over the Qwen3-8B layer matrices and small ones: each the
    row-major GPU codes (checked against the oracle elsewhere) permuted."""
    shapes = [(n, k) for _, n, k in LAYER_SHAPES_QWEN3_8B] + [(144, 384), (16, 128), (0, 256)]
    announce("frag weight quant multi", shapes)
    ws = [device_bf16_normal(sh, 0.02, seed=30 + i) if sh[0] else torch.empty(sh, dtype=torch.bfloat16, device="cuda")
          for i, sh in enumerate(shapes)]
    rows = fb.quantize_weights_blockwise_multi(ws)
    frags = fb.quantize_weights_blockwise_frag_multi(ws)
    for (q, s), (qf, sf), (n, k) in zip(rows, frags, shapes):
        if n == 0:
            continue
        perm = q.view(n // 16, 16, k // 128, 2, 4, 16).permute(0, 2, 3, 4, 1, 5).contiguous().view(n, k)
        assert torch.equal(qf, perm) and torch.equal(sf, s), (n, k)


def test_frag_shape_errors(fb):
    w = torch.zeros((24, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.quantize_weight_blockwise_frag(w)
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.quantize_weights_blockwise_frag_multi([torch.zeros((16, 200), dtype=torch.bfloat16, device="cuda")])
    a = torch.zeros((16, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.gemm_w8a8_blockscaled_frag(a, torch.ones((16, 2), device="cuda"), torch.zeros((24, 256), dtype=torch.uint8,
                                      device="cuda"), torch.ones((1, 2), device="cuda"))


def test_afrag_shape_errors(fb):
    a = torch.zeros((24, 256), dtype=torch.uint8, device="cuda")
    s = torch.ones((24, 2), device="cuda")
    with pytest.raises(fb.FP8BQError, match="shape"):
        fb.gemm_w8a8_blockscaled_afrag(a, s, a, torch.ones((1, 2), device="cuda"))
    with pytest.raises(ValueError):
        fb.quantize_act_per_token_group_frag(torch.zeros((24, 128), dtype=torch.bfloat16, device="cuda"))
