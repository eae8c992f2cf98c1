"""GPU parity of the two quantizers: bit-exact codes and scales vs the oracle.

Cases: the tiny configuration (384x512 weights, 32x512 activations with 4
outlier channels x50), ragged and unaligned shapes, special tiles (all-zero,
signed zeros, single element, constant, tiny amax taking the IEEE-divide
path, huge amax, exact E4M3 ties), per-block scale spreads, the Qwen3-8B
layer shapes, the 36-layer re-quantization sweep (sampled blocks), and the
prefill / MoE activation shapes (sampled rows).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import announce, bf16_bits_to_device
from synthetic import LAYER_SHAPES_QWEN3_8B, activations, bf16_normal, device_bf16_normal, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def gpu_quant_weight(fb, bits):
    q, s = fb.quantize_weight_blockwise(bf16_bits_to_device(bits))
    return q.cpu().numpy(), s.cpu().numpy()


def gpu_quant_act(fb, bits):
    q, s = fb.quantize_act_per_token_group(bf16_bits_to_device(bits))
    return q.cpu().numpy(), s.cpu().numpy()


def assert_same(got, want, what):
    gq, gs = got
    wq, ws = want
    assert gs.shape == ws.shape, (what, gs.shape, ws.shape)
    bad_s = np.nonzero(gs.view(np.uint32) != ws.view(np.uint32))
    assert bad_s[0].size == 0, (what, "scales differ", [x[:5] for x in bad_s])
    bad_q = np.nonzero(gq != wq)
    assert bad_q[0].size == 0, (what, "codes differ", bad_q[0].size, [x[:5] for x in bad_q],
                                gq[bad_q][:5], wq[bad_q][:5])


# ---------------------------------------------------------------- weights

def test_weight_tiny_config(fb):
    announce("quant_weight tiny 384x512")
    w = bf16_normal((384, 512), 0.02, (1, 0, 0))
    assert_same(gpu_quant_weight(fb, w), oracle.quant_weight_blockwise(w), "tiny")


@pytest.mark.parametrize("shape", [(200, 300), (1, 1), (129, 127), (5, 1001), (130, 260), (128, 8), (3, 128)])
def test_weight_ragged_shapes(fb, shape):
    announce("quant_weight ragged", shape)
    w = bf16_normal(shape, 0.02, (2, *shape))
    assert_same(gpu_quant_weight(fb, w), oracle.quant_weight_blockwise(w), shape)


def test_weight_batched(fb):
    announce("quant_weight batch 3 x 256x384")
    w = bf16_normal((3, 256, 384), 0.02, (3, 0))
    assert_same(gpu_quant_weight(fb, w), oracle.quant_weight_blockwise(w), "batch")


def _special_matrix():
    """A 512x512 matrix whose 16 blocks each hold one special case."""
    rng = np.random.default_rng(11)
    x = np.zeros((512, 512), np.float32)
    blocks = {}
    z = rng.standard_normal((128, 128)).astype(np.float32)
    blocks[(0, 0)] = np.zeros((128, 128), np.float32)  # all zero (some -0 below)
    b = np.zeros((128, 128), np.float32)
    b[7, 9] = -0.37
    blocks[(0, 1)] = b  # single element
    blocks[(0, 2)] = np.full((128, 128), 1.7, np.float32)  # constant
    blocks[(0, 3)] = z * np.float32(2.0 ** -130)  # bf16 denormals: denormal scale, IEEE path
    blocks[(1, 0)] = z * np.float32(1e-20)  # s < 2^-64: IEEE path, normal scale
    blocks[(1, 1)] = z * np.float32(3e-17)  # just above the fast-path threshold
    blocks[(1, 2)] = z * np.float32(1e36)  # huge amax
    ties = np.array([448, -1, 0.5, 3, -240, 2 ** -6, 2 ** -9, 1.0625, 1.1875, 400, 432, 7.5 * 2 ** -9, 2 ** -10],
                    np.float32)
    blocks[(1, 3)] = rng.choice(ties, (128, 128)).astype(np.float32)  # exact E4M3 ties at s = 1
    blocks[(1, 3)][0, 0] = 448
    for i in range(2, 4):
        for j in range(4):
            blocks[(i, j)] = z * np.float32(2.0 ** rng.integers(-40, 40)) * rng.uniform(0.5, 2)
    for (i, j), v in blocks.items():
        x[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = v
    bits = f32_to_bf16_bits(x)
    bits[3:10, 5] |= 0x8000  # negative zeros in the all-zero block
    return bits


def test_weight_special_blocks(fb):
    announce("quant_weight special blocks")
    w = _special_matrix()
    got = gpu_quant_weight(fb, w)
    want = oracle.quant_weight_blockwise(w)
    assert_same(got, want, "special")
    assert want[1][0, 0] == 0 and got[0][3, 5] == 0x80


def test_weight_scale_spread(fb):
    announce("quant_weight per-block scale spread")
    rng = np.random.default_rng(12)
    z = rng.standard_normal((1024, 1024)).astype(np.float32)
    mult = np.exp2(rng.uniform(-60, 60, (8, 8))).astype(np.float32)
    x = z * np.kron(mult, np.ones((128, 128), np.float32))
    w = f32_to_bf16_bits(x)
    assert_same(gpu_quant_weight(fb, w), oracle.quant_weight_blockwise(w), "spread")


@pytest.mark.parametrize("idx", range(len(LAYER_SHAPES_QWEN3_8B)))
def test_weight_qwen3_8b_layer(fb, idx):
    name, n, k = LAYER_SHAPES_QWEN3_8B[idx]
    announce("quant_weight qwen3-8b", name, n, k)
    w = bf16_normal((n, k), 0.02, (4, idx))
    gq, gs = gpu_quant_weight(fb, w)
    if n * k <= 4096 * 4096:
        assert_same((gq, gs), oracle.quant_weight_blockwise(w), name)
        return
    rng = np.random.default_rng(5)
    for _ in range(48):
        i, j = int(rng.integers(0, n // 128)), int(rng.integers(0, k // 128))
        blk = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
        q, s = oracle.quant_weight_block(w[blk])
        assert gs[i, j].view(np.uint32) == np.float32(s).view(np.uint32), (name, i, j)
        assert np.array_equal(gq[blk], q), (name, i, j)


def _oracle_quant_rows(bits):
    """oracle.quant_weight_blockwise of [N][K] bits, one 128-row block row per
    task on a thread pool (blocks are independent)."""
    from concurrent.futures import ThreadPoolExecutor

    chunks = [(r, min(bits.shape[0], r + 128)) for r in range(0, bits.shape[0], 128)]
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(lambda c: oracle.quant_weight_blockwise(bits[c[0]:c[1]]), chunks))
    return np.concatenate([q for q, _ in res]), np.concatenate([s for _, s in res])


def test_weight_36_layer_sweep_sampled(fb):
    """Full-size re-quantization sweep (36 layers x 4 projections, batch = 36
    per call): the last layer of every projection in full (its bytes lie
    past 2^31 in the batched call) and random blocks of the others."""
    rng = np.random.default_rng(6)
    for p, (name, n, k) in enumerate(LAYER_SHAPES_QWEN3_8B):
        announce("quant_weight sweep", name, 36, n, k)
        w = device_bf16_normal((36, n, k), 0.02, seed=1000 + p)
        q, s = fb.quantize_weight_blockwise(w)
        torch.cuda.synchronize()
        oq, os_ = _oracle_quant_rows(w[35].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(s[35].cpu().numpy().view(np.uint32), os_.view(np.uint32)), (name, "layer 35 scales")
        assert np.array_equal(q[35].cpu().numpy(), oq), (name, "layer 35 codes")
        for _ in range(6):
            l, i, j = int(rng.integers(0, 36)), int(rng.integers(0, n // 128)), int(rng.integers(0, k // 128))
            blk = w[l, i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].contiguous().view(torch.int16)
            oq, os_ = oracle.quant_weight_block(blk.cpu().numpy().view(np.uint16))
            got_s = s[l, i, j].reshape(1).cpu().numpy()
            assert got_s.view(np.uint32)[0] == np.float32(os_).view(np.uint32), (name, l, i, j)
            assert np.array_equal(q[l, i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].cpu().numpy(), oq)
        del w, q, s
        torch.cuda.empty_cache()


# ------------------------------------------------------------ activations

def test_act_tiny_config(fb):
    announce("quant_act tiny 32x512 outliers x50")
    x, _ = activations(32, 512, (1, 1, 0), n_outliers=4, outlier_mult=50.0)
    assert_same(gpu_quant_act(fb, x), oracle.quant_act_per_token_group(x), "tiny")


@pytest.mark.parametrize("shape", [(7, 300), (1, 1), (3, 1001), (5, 8), (2, 130), (1, 128), (33, 4100)])
def test_act_ragged_shapes(fb, shape):
    announce("quant_act ragged", shape)
    x, _ = activations(*shape, (2, *shape), n_outliers=1, outlier_mult=30.0)
    assert_same(gpu_quant_act(fb, x), oracle.quant_act_per_token_group(x), shape)


def test_act_special_groups(fb):
    announce("quant_act special groups")
    w = _special_matrix()  # reuse: rows of 512 = 4 groups, many special values
    assert_same(gpu_quant_act(fb, w), oracle.quant_act_per_token_group(w), "special")


@pytest.mark.parametrize("k", [4096, 12288])
def test_act_decode_shapes(fb, k):
    announce("quant_act decode 256 x", k)
    x, _ = activations(256, k, (3, k))
    assert_same(gpu_quant_act(fb, x), oracle.quant_act_per_token_group(x), k)


@pytest.mark.parametrize("k,n_out", [(4096, 41), (12288, 123)])
def test_act_prefill_shapes_sampled_rows(fb, k, n_out):
    announce("quant_act prefill 8192 x", k)
    x, _ = activations(8192, k, (4, k), n_outliers=n_out, outlier_mult=30.0)
    gq, gs = gpu_quant_act(fb, x)
    rows = np.sort(np.random.default_rng(k).choice(8192, 512, replace=False))
    wq, ws = oracle.quant_act_per_token_group(x[rows])
    assert_same((gq[rows], gs[rows]), (wq, ws), k)


def test_act_moe_shape_sampled_rows(fb):
    announce("quant_act moe 32768 x 2048")
    x, _ = activations(32768, 2048, (5, 0))
    gq, gs = gpu_quant_act(fb, x)
    rows = np.sort(np.random.default_rng(9).choice(32768, 1024, replace=False))
    assert_same((gq[rows], gs[rows]), oracle.quant_act_per_token_group(x[rows]), "moe")


def test_act_empty(fb):
    announce("quant_act empty")
    q, s = fb.quantize_act_per_token_group(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    q, s = fb.quantize_weight_blockwise(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_weights_multi_matches_single():
    """quantize_weights_blockwise_multi: one launch over matrices of any shapes
    (full Qwen3-8B layer shapes, ragged edges, K % 8 != 0, empty) gives each
    one the oracle's codes and scales."""
    import fp8_blockwise_quantized_quantize_amd as fb

    shapes = [(n, k) for _, n, k in LAYER_SHAPES_QWEN3_8B] + [(200, 136), (37, 300), (1, 8), (0, 128), (130, 129)]
    announce("weights multi", shapes)
    ws_bits = [bf16_normal(sh, 0.02, (140 + i, 0, 0)) if sh[0] * sh[1] else np.zeros(sh, np.uint16)
               for i, sh in enumerate(shapes)]
    ws = [torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16) for b in ws_bits]
    res = fb.quantize_weights_blockwise_multi(ws)
    torch.cuda.synchronize()
    for (q, s), b, sh in zip(res, ws_bits, shapes):
        if sh[0] * sh[1] == 0:
            continue
        rq, rs = oracle.quant_weight_blockwise(b)
        assert np.array_equal(q.cpu().numpy(), rq), sh
        assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), sh


def test_acts_multi_matches_oracle(fb):
    """quantize_acts_per_token_group_multi: one launch over the four decode
    activations of a Qwen3-8B layer (M = 256; K = 4096 x 3 and 12288) plus
    ragged shapes (K % 8 != 0, a partial last group, one row, empty) gives
    each one the oracle's codes and scales."""
    shapes = [(256, k) for _, _, k in LAYER_SHAPES_QWEN3_8B] + [(7, 300), (1, 1), (33, 4100), (0, 256), (5, 8)]
    announce("acts multi", shapes)
    xs_bits = []
    for i, (m, k) in enumerate(shapes):
        if m * k == 0:
            xs_bits.append(np.zeros((m, k), np.uint16))
        else:
            xs_bits.append(activations(m, k, (150 + i, 0), n_outliers=min(4, k), outlier_mult=50.0)[0])
    xs = [bf16_bits_to_device(b) for b in xs_bits]
    res = fb.quantize_acts_per_token_group_multi(xs)
    torch.cuda.synchronize()
    for (q, s), b, sh in zip(res, xs_bits, shapes):
        if sh[0] * sh[1] == 0:
            continue
        assert_same((q.cpu().numpy(), s.cpu().numpy()), oracle.quant_act_per_token_group(b), ("acts multi", sh))


def test_acts_multi_limits(fb):
    x = torch.zeros((2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fb.quantize_acts_per_token_group_multi([x] * (fb.MAX_ACT_DESCS + 1))
    assert fb.quantize_acts_per_token_group_multi([]) == []
