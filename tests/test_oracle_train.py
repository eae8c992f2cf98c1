"""Pins of the training-quantization oracle (oracle/train.py): W^T's blocks
are W's blocks transposed; x^T's groups along M are columns of x; the
dequantized wgrad operand reconstructs x within the group error bound."""

import numpy as np
import pytest

from oracle import decode_e4m3, quant_act_per_token_group, quant_weight_blockwise
from oracle.bf16 import bf16_bits_to_f32
from oracle.train import quant_act_dual, quant_weight_blockwise_dual
from synthetic import bf16_normal, f32_to_bf16_bits


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (200, 130), (37, 300), (1, 129)])
def test_weight_transpose_is_the_transposed_blocks(N, K):
    w = bf16_normal((N, K), 0.02, (120, N, K))
    (q, s), (qt, st) = quant_weight_blockwise_dual(w)
    assert qt.shape == (K, N) and st.shape == s.T.shape
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_weight_dual_batched():
    w = bf16_normal((3, 256, 128), 0.02, (121, 0, 0))
    (q, s), (qt, st) = quant_weight_blockwise_dual(w)
    for b in range(3):
        q1, s1 = quant_weight_blockwise(w[b])
        assert np.array_equal(q[b], q1) and np.array_equal(qt[b], q1.T) and np.array_equal(st[b], s1.T)


@pytest.mark.parametrize("M,K", [(128, 128), (300, 256), (77, 200), (1, 128), (129, 8)])
def test_act_transposed_groups_run_along_tokens(M, K):
    rng = np.random.default_rng([122, M, K])
    z = rng.normal(0, 1, (M, K)).astype(np.float32)
    z[:, rng.integers(0, K)] *= 30.0                          # an outlier channel
    x = f32_to_bf16_bits(z)
    (q, s), (qt, st) = quant_act_dual(x)
    assert q.shape == (M, K) and qt.shape == (K, M) and st.shape == (K, -(-M // 128))
    xf = bf16_bits_to_f32(x)
    # the scale of group g of channel k is max |x[128 g : 128 g + 128, k]| / 448
    for k in (0, K // 2, K - 1):
        for g in range(st.shape[1]):
            col = xf[128 * g:128 * g + 128, k]
            assert st[k, g] == np.float32(np.abs(col).max() / np.float32(448))
    # each row of x^T's codes is channel k quantized like a token
    q1, s1 = quant_act_per_token_group(np.ascontiguousarray(x[:, :1].T))
    assert np.array_equal(qt[:1], q1) and np.array_equal(st[:1], s1)
    # the forward half is the per-token quantizer
    q0, s0 = quant_act_per_token_group(x)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)


def test_act_transposed_reconstruction_bound():
    rng = np.random.default_rng(123)
    x = f32_to_bf16_bits(rng.normal(0, 1, (256, 128)).astype(np.float32))
    _, (qt, st) = quant_act_dual(x)
    xf = bf16_bits_to_f32(x).T.astype(np.float64)
    sv = np.repeat(st.astype(np.float64), 128, axis=1)[:, :256]
    err = np.abs(decode_e4m3(qt) * sv - xf)
    assert np.all(err <= (2.0 ** -4 + 2.0 ** -23) * np.abs(xf) + 2.0 ** -10 * sv + 1e-30)
