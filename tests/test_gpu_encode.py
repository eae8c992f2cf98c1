"""GPU: the library's E4M3 conversion against the oracle over every float32.

Expected codes are the oracle's: its encoder is a step function of the
float32 bit pattern, determined by the 126 transition points that
helpers.e4m3_transition_table finds with the oracle's encoder (that
expansion is itself checked against the oracle in test_transition_table.py).
"""

import numpy as np
import pytest
import torch

from helpers import announce, e4m3_transition_table

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
F32_464 = 0x43E80000  # bits of 464.0
F32_INF = 0x7F800000


@pytest.fixture(scope="module")
def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


@pytest.fixture(scope="module")
def table():
    return torch.from_numpy(e4m3_transition_table().astype(np.int32)).cuda()


def _sweep(fb, table, method, mag_end):
    bad = 0
    first = []
    for neg in (False, True):
        for lo in range(0, mag_end, CHUNK):
            hi = min(mag_end, lo + CHUNK)
            mag = torch.arange(lo, hi, dtype=torch.int32, device="cuda")
            bits = mag | torch.tensor(-(2 ** 31), dtype=torch.int32, device="cuda") if neg else mag
            got = fb.encode_e4m3(bits.view(torch.float32), method=method)
            want = torch.searchsorted(table, mag, right=True, out_int32=True).to(torch.uint8)
            if neg:
                want |= 0x80
            ne = got != want
            n = int(ne.sum())
            if n:
                bad += n
                idx = torch.nonzero(ne)[:4, 0]
                first += [(hex(int(bits[i]) & 0xFFFFFFFF), int(got[i]), int(want[i])) for i in idx]
            del mag, bits, got, want, ne
    torch.cuda.synchronize()
    return bad, first


def test_hardware_conversion_in_quantizer_range(fb, table):
    announce("encode method 0 (hardware, |v| < 464), every float32")
    bad, first = _sweep(fb, table, 0, F32_464)
    assert bad == 0, first


def test_saturating_encoder_all_finite(fb, table):
    announce("encode method 1 (clamp + hardware), every finite float32")
    bad, first = _sweep(fb, table, 1, F32_INF)
    assert bad == 0, first


def test_integer_encoder_all_finite(fb, table):
    announce("encode method 2 (integer bits), every finite float32")
    bad, first = _sweep(fb, table, 2, F32_INF)
    assert bad == 0, first


def test_hand_values(fb):
    from test_oracle_e4m3 import load_hand_table

    rows = load_hand_table()
    v = torch.tensor([r[0] for r in rows], dtype=torch.float32, device="cuda")
    want = [r[1] for r in rows]
    for method in (1, 2):
        got = fb.encode_e4m3(v, method=method).cpu().tolist()
        assert got == want, (method, got)
