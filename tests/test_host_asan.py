"""The C-ABI layer's host code under AddressSanitizer (CPU only).

The library is built once more with AddressSanitizer on its host code only
(every sanitizer flag is given to the host compilation pass; device code is
the same), and a child process with the ASan runtime preloaded calls every
entry point through ctypes with arguments the host checks must reject:
null and misaligned pointers, negative, overflowing and non-multiple-of-128
sizes, descriptor arrays at and past their limits (the host loops over them
are the code most exposed to out-of-bounds reads), unknown tiles and modes,
and the status strings of every code.  Without a GPU each call that passes
its checks stops at the device check.  ASan aborts the child on any invalid
host memory access.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join("/tmp", "fp8bq_host_asan", "libfp8bq_asan.so")


def _asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib():
    if not os.path.exists(HIPCC) or _asan_runtime() is None:
        pytest.skip("hipcc or the ASan runtime is not available")
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_fp8bq_build", os.path.join(ROOT, "fp8_blockwise_quantized_quantize_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    srcs = mod.sources()
    newest = max(os.path.getmtime(p) for p in srcs + [os.path.join(ROOT, "include", "fp8bq.h")])
    if not os.path.exists(OUT) or os.path.getmtime(OUT) < newest:
        os.makedirs(os.path.dirname(OUT), exist_ok=True)
        host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                     "-shared-libsan"]
        cmd = [HIPCC, *mod.FLAGS, *host_asan, "-I", os.path.join(ROOT, "include"), "-o", OUT, *srcs]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-3000:]
    return OUT


CHILD = r'''
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
P, I, F, C = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
good, odd, null = P(4096), P(4097), P(0)
def call(name, argtypes, *args):
    f = getattr(lib, name)
    f.argtypes = argtypes
    f.restype = C
    return f(*args)
lib.fp8bq_status_string.argtypes = [C]
lib.fp8bq_status_string.restype = ctypes.c_char_p
for code in range(-1, 12):
    assert lib.fp8bq_status_string(code)
g8 = [P, P, P, P, P, I, I, I, P]
assert call("quantize_weight_blockwise", [P, P, P, I, I, I, P], good, good, good, 1, -1, 128, null) == 2
assert call("quantize_weight_blockwise", [P, P, P, I, I, I, P], null, good, good, 1, 8, 128, null) == 1
assert call("quantize_weight_blockwise", [P, P, P, I, I, I, P], odd, good, good, 1, 8, 128, null) == 3
assert call("quantize_weight_blockwise", [P, P, P, I, I, I, P], good, good, good, 1 << 40, 1 << 20, 1 << 20, null) == 2
assert call("quantize_act_per_token_group", [P, P, P, I, I, P], good, good, good, -5, 128, null) == 2
assert call("gemm_w8a8_blockscaled", g8, good, good, good, good, good, 4, 4, 100, null) == 2
assert call("gemm_w8a8_blockscaled", g8, good, good, good, good, odd, 4, 4, 128, null) == 3
assert call("gemm_w8a8_blockscaled_tile", g8[:8] + [C, P], good, good, good, good, good, 4, 4, 128, 99, null) == 6
assert call("gemm_w8a8_blockscaled_splitk", g8[:8] + [P, I, P], good, good, good, good, good, 4, 4, 100, null, 0,
            null) == 2
n = I(0)
assert call("gemm_w8a8_blockscaled_splitk_workspace", [I, I, I, ctypes.POINTER(I)], 4, 4, 100, ctypes.byref(n)) == 2
assert call("gemm_w8a8_blockscaled_splitk_workspace", [I, I, I, P], 4, 4, 128, null) == 1
assert call("gemm_w8a8_blockscaled_splitk_noalloc", g8, good, good, good, good, good, 4, 4, 100, null) == 2
assert call("gemm_w8a8_blockscaled_afrag", g8, good, good, good, good, good, 24, 4, 256, null) == 2
assert call("quantize_act_per_token_group_frag", [P, P, P, I, I, P], good, good, good, 24, 128, null) == 2
gg = [P, P, P, P, P, P, I, I, I, I, P]
assert call("grouped_gemm_w8a8_blockscaled", gg, good, good, good, good, good, good, 4, 4, 100, 2, null) == 2
assert call("grouped_gemm_w8a8_blockscaled", gg, good, good, good, good, good, good, 4, 4, 128, 0, null) == 2
gt = [P, P, I, P, I, P, P, P, P, I, I, I, I, C, P]
assert call("grouped_gemm_w8a8_blockscaled_tile", gt, good, good, 4, null, 1, good, good, good, good, 4, 4, 128, 2,
            1, null) == 6
assert call("grouped_gemm_w8a8_blockscaled_gather", gt[:13] + [P], good, good, 4, null, 1, good, good, good, good, 4,
            4, 128, 2, null) == 1
assert call("fp8bq_check_group_offsets", [P, I, I, P], good, 0, 4, null) == 2
assert call("fp8bq_encode_e4m3", [P, P, I, C, P], good, good, 8, 7, null) == 2

class WD(ctypes.Structure):
    _fields_ = [("w", P), ("q", P), ("s", P), ("N", I), ("K", I)]
for count in (0, 1, 48, 49):
    arr = (WD * max(count, 1))(*[WD(4096, 4096, 4096, 0, 0)] * max(count, 1))
    rc = call("quantize_weights_blockwise_multi", [ctypes.POINTER(WD), I, P], arr, count, null)
    assert rc == (2 if count > 48 else 0), (count, rc)
arr = (WD * 3)(WD(4096, 4096, 4096, 128, 128), WD(4096, 4096, 4097, 128, 128), WD(4096, 4096, 4096, 1, 1))
assert call("quantize_weights_blockwise_multi", [ctypes.POINTER(WD), I, P], arr, 3, null) == 3
for count in (0, 1, 16, 17):
    arr = (WD * max(count, 1))(*[WD(4096, 4096, 4096, 0, 0)] * max(count, 1))
    rc = call("quantize_acts_per_token_group_multi", [ctypes.POINTER(WD), I, P], arr, count, null)
    assert rc == (2 if count > 16 else 0), (count, rc)
arr = (WD * 2)(WD(4096, 4096, 4096, 2, 128), WD(null, 4096, 4096, 2, 128))
assert call("quantize_acts_per_token_group_multi", [ctypes.POINTER(WD), I, P], arr, 2, null) == 1
assert call("token_importance_weights", [P, P, P, P, P, P, I, F, C, P], good, good, null, null, good, null, 8, 0.5,
            0, null) == 6
assert call("moe_sort_by_expert", [P, I, I, I, P, P, P, P], good, 4, 2, 0, good, good, good, null) == 2
assert call("silu_mul_quantize_act", [P, I, I, P, P, P, P], good, 4, 12, good, good, null, null) == 2
assert call("moe_combine", [P, P, P, I, I, I, I, P, P], good, good, good, 4, 2, 12, 8, good, null) == 2
assert call("kv_scale_calibrate", [P, P, I, I, I, C, P, P, P], good, null, 4, 2, 64, 2, good, null, null) == 6
assert call("kv_cache_write_fp8", [P, P, P, P, P, C, P, P, I, I, I, I, P], good, null, good, good, null, 1, good,
            null, 4, 2, 64, -1, null) == 2
assert call("quantize_weight_blockwise_dual", [P, P, P, P, P, I, I, I, P], good, good, null, good, good, 1, 8, 128,
            null) == 6
assert call("quantize_act_dual", [P, P, P, P, P, I, I, P], good, good, good, good, good, 4, 12, null) == 2
print("asan host checks ok", flush=True)
'''


def test_host_code_under_address_sanitizer(asan_lib):
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", CHILD, asan_lib], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "asan host checks ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr
