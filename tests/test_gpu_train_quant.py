"""GPU parity of the FP8 training-operand quantizers (quantize_weight_blockwise_dual,
quantize_act_dual) against the oracle (oracle/train.py).  Bar: bit-exact
codes and scales in both layouts."""

import numpy as np
import pytest

from helpers import announce
from oracle.train import quant_act_dual, quant_weight_blockwise_dual
from synthetic import bf16_normal, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (200, 136), (37, 304), (1, 8), (3, 256, 128), (2, 130, 8)])
def test_weight_dual(shape):
    announce("weight dual", shape)
    w = bf16_normal(shape, 0.02, (130, *shape[-2:]))
    (q, s), (qt, st) = fb().quantize_weight_blockwise_dual(bf(w))
    (rq, rs), (rqt, rst) = quant_weight_blockwise_dual(w)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    assert np.array_equal(host(qt), rqt) and np.array_equal(host(st), rst)
    # and the forward half equals the plain weight quantizer
    q2, s2 = fb().quantize_weight_blockwise(bf(w))
    assert np.array_equal(host(q2), rq) and np.array_equal(host(s2), rs)
    # transposed only
    (n0, n1), (qt3, st3) = fb().quantize_weight_blockwise_dual(bf(w), forward=False)
    assert n0 is None and np.array_equal(host(qt3), rqt) and np.array_equal(host(st3), rst)


@pytest.mark.parametrize("M,K", [(128, 128), (300, 256), (77, 200), (1, 128), (129, 8), (256, 4096), (1000, 96)])
def test_act_dual(M, K):
    announce("act dual", M, K)
    rng = np.random.default_rng([131, M, K])
    z = rng.standard_normal((M, K), dtype=np.float32)
    z[:, rng.integers(0, K, max(1, K // 100))] *= 30.0       # outlier channels
    z[rng.integers(0, M)] *= 0.0                             # a zero token
    x = f32_to_bf16_bits(z)
    (q, s), (qt, st) = fb().quantize_act_dual(bf(x))
    (rq, rs), (rqt, rst) = quant_act_dual(x)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    assert np.array_equal(host(qt), rqt) and np.array_equal(host(st), rst)
    (_, _), (qt2, st2) = fb().quantize_act_dual(bf(x), forward=False)
    assert np.array_equal(host(qt2), rqt) and np.array_equal(host(st2), rst)


def test_act_dual_zero_channel_groups():
    # a channel that is zero over a whole 128-token group: scale 0, codes keep the zero's sign
    M, K = 256, 128
    x = f32_to_bf16_bits(np.random.default_rng(132).standard_normal((M, K), dtype=np.float32))
    x[:128, 5] = 0
    x[:128:2, 5] = 0x8000
    (q, s), (qt, st) = fb().quantize_act_dual(bf(x))
    (rq, rs), (rqt, rst) = quant_act_dual(x)
    assert np.array_equal(host(qt), rqt) and np.array_equal(host(st), rst)
    assert host(st)[5, 0] == 0 and np.all(host(qt)[5, :128:2] == 0x80)


def test_act_dual_training_microbatch_qwen3_8b():
    # the input of a Qwen3-8B layer for an 8192-token micro-batch, every byte compared
    M, K = 8192, 4096
    announce("act dual full", M, K)
    rng = np.random.default_rng(133)
    z = rng.standard_normal((M, K), dtype=np.float32)
    z[:, rng.choice(K, 41, replace=False)] *= 30.0
    x = f32_to_bf16_bits(z)
    (q, s), (qt, st) = fb().quantize_act_dual(bf(x))
    (rq, rs), (rqt, rst) = quant_act_dual(x)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    assert np.array_equal(host(qt), rqt) and np.array_equal(host(st), rst)
