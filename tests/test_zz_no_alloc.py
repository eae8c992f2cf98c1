"""The allocation-free K-split GEMM (gemm_w8a8_blockscaled_splitk_noalloc):
its partials go to the library's static device scratch instead of a caller
workspace.  Checked through the C ABI against the workspace entry point
(gemm_w8a8_blockscaled_splitk, same kernels: same bits) and the oracle, on
two calls in a row, the second on a smaller problem, so the second call
runs on scratch that still holds the first call's partials."""

import numpy as np
import pytest
import torch

import oracle
from helpers import announce, assert_gemm_close, device_to_bits
from synthetic import activations, bf16_normal

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, seed):
    x, _ = activations(m, k, (seed, 0), n_outliers=4, outlier_mult=30.0)
    w = bf16_normal((n, k), 0.02, (seed, 1))
    qa, sa = oracle.quant_act_per_token_group(x)
    qw, sw = oracle.quant_weight_blockwise(w)
    return qa, sa, qw, sw


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_equals_workspace_entry_on_two_calls_in_a_row():
    import fp8_blockwise_quantized_quantize_amd as fb

    for m, n, k in [(128, 4096, 12288), (33, 520, 9344)]:  # the second call is smaller
        announce("gemm split-K noalloc", m, n, k)
        need = fb.splitk_workspace_bytes(m, n, k)
        assert 0 < need <= 32 * 1024 * 1024  # the split runs, within the static scratch
        qa, sa, qw, sw = _inputs(m, n, k, 170 + m)
        a, s_a, w, s_w = _dev(qa), _dev(sa), _dev(qw), _dev(sw)
        y_ws = fb.gemm_w8a8_blockscaled_splitk(a, s_a, w, s_w,
                                               workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
        y_na = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        fb.gemm_w8a8_blockscaled_splitk_noalloc(a, s_a, w, s_w, y_na)
        got = device_to_bits(y_na)
        assert np.array_equal(got, device_to_bits(y_ws))
        print(assert_gemm_close(got, oracle.gemm_ref(qa, sa, qw, sw)))


def test_noalloc_unsplit_shape_and_errors():
    import fp8_blockwise_quantized_quantize_amd as fb

    announce("gemm split-K noalloc unsplit + errors")
    qa, sa, qw, sw = _inputs(512, 256, 512, 180)
    a, s_a, w, s_w = _dev(qa), _dev(sa), _dev(qw), _dev(sw)
    y_na = torch.empty((512, 256), dtype=torch.bfloat16, device="cuda")
    fb.gemm_w8a8_blockscaled_splitk_noalloc(a, s_a, w, s_w, y_na)
    assert torch.equal(y_na.view(torch.int16), fb.gemm_w8a8_blockscaled(a, s_a, w, s_w).view(torch.int16))
    with pytest.raises(fb.FP8BQError, match="shape"):
        lib = fb.raw_library()
        code = lib.gemm_w8a8_blockscaled_splitk_noalloc(a.data_ptr(), s_a.data_ptr(), w.data_ptr(), s_w.data_ptr(),
                                                         y_na.data_ptr(), 512, 256, 500, None)
        fb._check("gemm_w8a8_blockscaled_splitk_noalloc", code)
