"""GPU parity of the FP8 KV cache (kv_scale_calibrate, kv_cache_write_fp8)
against the oracle (oracle/kv.py).  Bar: scales and cache bytes bit-exact
(the scale is an exact max and one IEEE division; the codes are byte work);
slots not written keep their contents."""

import numpy as np
import pytest

from helpers import announce
from oracle.kv import kv_cache_write, kv_calibrate, kv_quantize
from oracle.bf16 import bf16_bits_to_f32
from synthetic import f32_to_bf16_bits

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
    return t.cpu().numpy()


def kv_bits(T, H, D, seed, std=1.0):
    rng = np.random.default_rng([110, seed])
    x = rng.standard_normal((T, H, D), dtype=np.float32) * np.float32(std)
    x *= rng.uniform(0.05, 8.0, (1, H, 1)).astype(np.float32)
    if T > 3:
        x[rng.integers(0, T, 3), rng.integers(0, H, 3), rng.integers(0, D, 3)] *= 40.0  # outliers
    return f32_to_bf16_bits(x)


def bf(a):
    return dev(a.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("T,H,D", [(0, 8, 128), (1, 1, 8), (7, 3, 64), (3000, 8, 128), (513, 64, 128), (100, 2, 8),
                                   (16384, 8, 128), (40, 16, 512)])
@pytest.mark.parametrize("per_head", [True, False])
def test_calibrate(T, H, D, per_head):
    announce("kv calibrate", T, H, D, per_head)
    k, v = kv_bits(T, H, D, 1), kv_bits(T, H, D, 2, std=0.3)
    ks, vs = fb().kv_scale_calibrate(bf(k), bf(v), per_head=per_head)
    if T == 0:
        assert np.all(host(ks) == 0) and np.all(host(vs) == 0)
        return
    assert np.array_equal(host(ks), kv_calibrate(k, per_head))
    assert np.array_equal(host(vs), kv_calibrate(v, per_head))
    # K alone
    ks2, vs2 = fb().kv_scale_calibrate(bf(k), None, per_head=per_head)
    assert vs2 is None and np.array_equal(host(ks2), host(ks))


@pytest.mark.parametrize("T,H,D,S", [(1, 1, 8, 4), (9, 2, 16, 20), (1000, 8, 128, 1500), (77, 64, 128, 100),
                                     (4099, 8, 128, 5000)])
@pytest.mark.parametrize("per_head", [True, False])
def test_cache_write(T, H, D, S, per_head):
    """Random slots with padding (-1 and S); the last shape is large enough
    for the four-chunks-per-lane kernel (524,672 chunks) with a ragged last
    workgroup."""
    announce("kv write", T, H, D, S, per_head)
    rng = np.random.default_rng([111, T])
    k, v = kv_bits(T, H, D, 3), kv_bits(T, H, D, 4)
    ks, vs = kv_calibrate(k, per_head), kv_calibrate(v, per_head)
    slots = rng.permutation(S)[:T].astype(np.int32)
    if T > 2:
        slots[0] = -1      # padding
        slots[T // 2] = S  # padding past the end
    kc = torch.full((S, H, D), 0xAB, dtype=torch.uint8, device=DEV)
    vc = torch.full((S, H, D), 0xCD, dtype=torch.uint8, device=DEV)
    fb().kv_cache_write_fp8(bf(k), bf(v), dev(slots), dev(ks), dev(vs), kc, vc)
    ref_k = kv_cache_write(np.full((S, H, D), 0xAB, np.uint8), k, ks, per_head, slots)
    ref_v = kv_cache_write(np.full((S, H, D), 0xCD, np.uint8), v, vs, per_head, slots)
    assert np.array_equal(host(kc), ref_k) and np.array_equal(host(vc), ref_v)


def test_saturation_and_zero_scale():
    T, H, D = 64, 4, 32
    k = kv_bits(T, H, D, 5)
    ks = kv_calibrate(k, True)
    big = f32_to_bf16_bits(np.float32(5.0) * bf16_bits_to_f32(k))   # beyond the calibrated range
    ks0 = ks.copy()
    ks0[1] = 0.0                                                       # an all-zero calibration head
    slots = np.arange(T, dtype=np.int32)
    for x, s in ((big, ks), (big, ks0), (k, ks0)):
        announce("kv saturation", float(s[1]))
        kc = torch.zeros((T, H, D), dtype=torch.uint8, device=DEV)
        fb().kv_cache_write_fp8(bf(x), None, dev(slots), dev(s), None, kc)
        ref = kv_quantize(x, s, True)
        assert np.array_equal(host(kc), ref)
    assert np.any((ref & 0x7F) == 0x7E)


def test_prefill_chunk_then_decode_writes_qwen3_8b():
    # one rollout's first forward (a 16384-token prefill chunk) calibrates the
    # layer's scales and fills the cache; 1536 decode tokens (one per
    # sequence of the rollout batch) then write with the same scales
    H, D = 8, 128
    T, S = 16384, 16384 + 1536 * 4
    k, v = kv_bits(T, H, D, 6), kv_bits(T, H, D, 7, std=0.5)
    announce("kv prefill", T, H, D)
    kd, vd = bf(k), bf(v)
    ks, vs = fb().kv_scale_calibrate(kd, vd, per_head=True)
    rks, rvs = kv_calibrate(k, True), kv_calibrate(v, True)
    assert np.array_equal(host(ks), rks) and np.array_equal(host(vs), rvs)
    kc = torch.zeros((S, H, D), dtype=torch.uint8, device=DEV)
    vc = torch.zeros((S, H, D), dtype=torch.uint8, device=DEV)
    slots = np.arange(T, dtype=np.int32)
    fb().kv_cache_write_fp8(kd, vd, dev(slots), ks, vs, kc, vc)
    assert np.array_equal(host(kc)[:T], kv_quantize(k, rks, True))
    assert np.array_equal(host(vc)[:T], kv_quantize(v, rvs, True))
    announce("kv decode", 1536)
    kn, vn = kv_bits(1536, H, D, 8, std=1.5), kv_bits(1536, H, D, 9, std=1.5)  # later steps: wider values
    dslots = (T + np.arange(1536) * 4 + 1).astype(np.int32)
    fb().kv_cache_write_fp8(bf(kn), bf(vn), dev(dslots), ks, vs, kc, vc)
    kh, vh = host(kc), host(vc)
    assert np.array_equal(kh[dslots], kv_quantize(kn, rks, True))
    assert np.array_equal(vh[dslots], kv_quantize(vn, rvs, True))
    untouched = np.setdiff1d(np.arange(T, S), dslots)
    assert np.all(kh[untouched] == 0) and np.all(vh[untouched] == 0)
