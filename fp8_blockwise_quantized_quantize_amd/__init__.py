"""Python binding of libfp8bq.so: blockwise W8A8 FP8 for AMD MI355X (gfx950).

Thin ctypes marshalling only: every function checks tensor dtypes, shapes,
devices and contiguity, allocates missing outputs with torch, and passes raw
device pointers plus torch's current HIP stream to the C ABI declared in
``include/fp8bq.h``.  All arithmetic runs in the library's HIP kernels; there
is no CPU fallback, and importing this package fails loudly when the built
library is missing (build it with ``python
fp8_blockwise_quantized_quantize_amd/build.py``).

The operations follow "FP8-RL: A Practical and Stable Low-Precision Stack for
LLM Reinforcement Learning" (paper-graph-ui summary page): §3.4.1 (E4M3,
128x128 weight blocks, 1x128 activation tiles, W^ = round(W / scale)) and
§3.4.2 (per-step weight re-quantization; FP8 GEMM with FP32 accumulation and
BF16 output).
"""

import ctypes
import os

import torch

__all__ = [
    "BLOCK",
    "LIB_PATH",
    "FP8BQError",
    "quantize_weight_blockwise",
    "quantize_weights_blockwise_multi",
    "quantize_weight_blockwise_frag",
    "quantize_weights_blockwise_frag_multi",
    "quantize_act_per_token_group",
    "quantize_acts_per_token_group_multi",
    "quantize_acts_per_token_group_frag_multi",
    "quantize_act_per_token_group_frag",
    "gemm_w8a8_blockscaled",
    "gemm_w8a8_blockscaled_splitk",
    "gemm_w8a8_blockscaled_splitk_noalloc",
    "splitk_workspace_bytes",
    "gemm_w8a8_blockscaled_afrag",
    "gemm_w8a8_blockscaled_frag",
    "grouped_gemm_w8a8_blockscaled",
    "grouped_gemm_w8a8_blockscaled_gather",
    "grouped_gemm_w8a8_blockscaled_gather_silu",
    "check_group_offsets",
    "TILES",
    "encode_e4m3",
    "token_importance_weights",
    "moe_sort_by_expert",
    "moe_gather_quantize_act",
    "silu_mul_quantize_act",
    "moe_combine",
    "moe_expert_ffn",
    "kv_scale_calibrate",
    "kv_cache_write_fp8",
    "quantize_weight_blockwise_dual",
    "quantize_act_dual",
    "status_string",
]

BLOCK = 128
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8bq.so")

# exported symbols of include/fp8bq.h
EXPORTS = (
    "fp8bq_status_string",
    "quantize_weight_blockwise",
    "quantize_weights_blockwise_multi",
    "quantize_weight_blockwise_frag",
    "quantize_weights_blockwise_frag_multi",
    "quantize_act_per_token_group",
    "quantize_acts_per_token_group_multi",
    "quantize_acts_per_token_group_frag_multi",
    "quantize_act_per_token_group_frag",
    "gemm_w8a8_blockscaled",
    "gemm_w8a8_blockscaled_frag",
    "gemm_w8a8_blockscaled_splitk",
    "gemm_w8a8_blockscaled_splitk_workspace",
    "gemm_w8a8_blockscaled_splitk_noalloc",
    "gemm_w8a8_blockscaled_afrag",
    "grouped_gemm_w8a8_blockscaled",
    "grouped_gemm_w8a8_blockscaled_gather",
    "grouped_gemm_w8a8_blockscaled_gather_silu",
    "gemm_w8a8_blockscaled_tile",
    "grouped_gemm_w8a8_blockscaled_tile",
    "fp8bq_check_group_offsets",
    "fp8bq_encode_e4m3",
    "token_importance_weights",
    "moe_sort_by_expert",
    "moe_gather_quantize_act",
    "silu_mul_quantize_act",
    "moe_combine",
    "kv_scale_calibrate",
    "kv_cache_write_fp8",
    "quantize_weight_blockwise_dual",
    "quantize_act_dual",
)


class FP8BQError(RuntimeError):
    pass


MAX_WEIGHT_DESCS = 48  # FP8BQ_MAX_WEIGHT_DESCS
MAX_ACT_DESCS = 16  # FP8BQ_MAX_ACT_DESCS


class _WeightDesc(ctypes.Structure):
    _fields_ = [("w_bf16", ctypes.c_void_p), ("w_fp8", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _ActDesc(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("x_fp8", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python fp8_blockwise_quantized_quantize_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fp8bq_status_string.argtypes = [i32]
    lib.fp8bq_status_string.restype = ctypes.c_char_p
    lib.quantize_weight_blockwise.argtypes = [p, p, p, i64, i64, i64, p]
    lib.quantize_act_per_token_group.argtypes = [p, p, p, i64, i64, p]
    lib.quantize_weights_blockwise_multi.argtypes = [ctypes.POINTER(_WeightDesc), i64, p]
    lib.quantize_weight_blockwise_frag.argtypes = [p, p, p, i64, i64, i64, p]
    lib.quantize_weights_blockwise_frag_multi.argtypes = [ctypes.POINTER(_WeightDesc), i64, p]
    lib.gemm_w8a8_blockscaled_frag.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.quantize_acts_per_token_group_multi.argtypes = [ctypes.POINTER(_ActDesc), i64, p]
    lib.quantize_acts_per_token_group_frag_multi.argtypes = [ctypes.POINTER(_ActDesc), i64, p]
    lib.gemm_w8a8_blockscaled.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.quantize_act_per_token_group_frag.argtypes = [p, p, p, i64, i64, p]
    lib.gemm_w8a8_blockscaled_afrag.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.grouped_gemm_w8a8_blockscaled.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, p]
    lib.grouped_gemm_w8a8_blockscaled_gather.argtypes = [p, p, i64, p, i64, p, p, p, p, i64, i64, i64, i64, p]
    lib.grouped_gemm_w8a8_blockscaled_gather_silu.argtypes = [p, p, i64, p, i64, p, p, p, p, p, i64, i64, i64, i64, p]
    lib.gemm_w8a8_blockscaled_tile.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p]
    lib.gemm_w8a8_blockscaled_splitk.argtypes = [p, p, p, p, p, i64, i64, i64, p, i64, p]
    lib.gemm_w8a8_blockscaled_splitk_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    lib.gemm_w8a8_blockscaled_splitk_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.grouped_gemm_w8a8_blockscaled_tile.argtypes = [p, p, i64, p, i64, p, p, p, p, i64, i64, i64, i64, i32, p]
    lib.fp8bq_check_group_offsets.argtypes = [p, i64, i64, p]
    lib.fp8bq_encode_e4m3.argtypes = [p, p, i64, i32, p]
    lib.token_importance_weights.argtypes = [p, p, p, p, p, p, i64, ctypes.c_float, i32, p]
    lib.moe_sort_by_expert.argtypes = [p, i64, i64, i64, p, p, p, p]
    lib.moe_gather_quantize_act.argtypes = [p, p, i64, i64, i64, i64, p, p, p]
    lib.silu_mul_quantize_act.argtypes = [p, i64, i64, p, p, p, p]
    lib.moe_combine.argtypes = [p, p, p, i64, i64, i64, i64, p, p]
    lib.kv_scale_calibrate.argtypes = [p, p, i64, i64, i64, i32, p, p, p]
    lib.kv_cache_write_fp8.argtypes = [p, p, p, p, p, i32, p, p, i64, i64, i64, i64, p]
    lib.quantize_weight_blockwise_dual.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.quantize_act_dual.argtypes = [p, p, p, p, p, i64, i64, p]
    for name in EXPORTS[1:]:
        getattr(lib, name).restype = i32
    return lib


_lib = _load()


def status_string(code):
    return _lib.fp8bq_status_string(int(code)).decode()


def _check(name, code):
    if code != 0:
        raise FP8BQError(f"{name}: {status_string(code)} (status {code})")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _require(t, name, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _u16(t):
    """BF16 tensors are passed by their bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)


def _cdiv(a, b):
    return -(-a // b)


# Tile kernels of the GEMMs by name (FP8BQ_TILE_* of the C ABI), for tests
# and diagnostics; None (or "auto") is the library's own choice.
TILES = {"auto": 0, "skinny64": 1, "skinny48": 2, "wide": 3, "decode_panel": 4, "deep": 5, "panel192": 6,
         "deep_persistent": 7, "skinny96": 8}


def _tile_id(tile):
    if tile is None:
        return 0
    if tile not in TILES:
        raise ValueError(f"unknown tile {tile!r}; one of {sorted(TILES)}")
    return TILES[tile]


def quantize_weight_blockwise(w, out=None, scale=None, frag=False):
    """BF16 weights [N, K] or [B, N, K] -> (E4M3 codes uint8, same shape; float32 scales [.., N/128, K/128]).
    ``frag``: codes in MFMA fragment order (quantize_weight_blockwise_frag; N % 16 == 0, K % 128 == 0)."""
    if w.dim() not in (2, 3):
        raise ValueError("weights must be [N, K] or [B, N, K]")
    b, n, k = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    _require(w, "w", _BF16, w.shape)
    sshape = (*w.shape[:-2], _cdiv(n, BLOCK), _cdiv(k, BLOCK))
    if out is None:
        out = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(sshape, dtype=torch.float32, device=w.device)
    _require(out, "out", _U8, w.shape, w.device)
    _require(scale, "scale", torch.float32, sshape, w.device)
    name = "quantize_weight_blockwise_frag" if frag else "quantize_weight_blockwise"
    with torch.cuda.device(w.device):
        _check(name, getattr(_lib, name)(_ptr(w), _ptr(out), _ptr(scale), b, n, k, _stream(w)))
    return out, scale


def quantize_weight_blockwise_frag(w, out=None, scale=None):
    """quantize_weight_blockwise with the codes in MFMA fragment order (N % 16 == 0, K % 128 == 0)."""
    return quantize_weight_blockwise(w, out, scale, frag=True)


def quantize_weights_blockwise_multi(ws, outs=None, frag=False):
    """Several BF16 matrices [N, K] (any shapes) in one launch -> list of (codes, scales),
    each exactly what quantize_weight_blockwise gives it (``frag``: what
    quantize_weight_blockwise_frag gives it).  ``outs``: optional list of (codes, scales) to fill."""
    ws = list(ws)
    if len(ws) > MAX_WEIGHT_DESCS:
        raise ValueError(f"at most {MAX_WEIGHT_DESCS} matrices per call")
    if not ws:
        return []
    dev = ws[0].device
    res = []
    descs = (_WeightDesc * len(ws))()
    for i, w in enumerate(ws):
        if w.dim() != 2:
            raise ValueError("each weight must be [N, K]")
        n, k = w.shape
        _require(w, f"w[{i}]", _BF16, (n, k), dev)
        if outs is None:
            q = torch.empty((n, k), dtype=torch.uint8, device=dev)
            s = torch.empty((_cdiv(n, BLOCK), _cdiv(k, BLOCK)), dtype=torch.float32, device=dev)
        else:
            q, s = outs[i]
        _require(q, f"out[{i}]", _U8, (n, k), dev)
        _require(s, f"scale[{i}]", torch.float32, (_cdiv(n, BLOCK), _cdiv(k, BLOCK)), dev)
        descs[i] = _WeightDesc(_ptr(_u16(w)).value, _ptr(q).value, _ptr(s).value, n, k)
        res.append((q, s))
    name = "quantize_weights_blockwise_frag_multi" if frag else "quantize_weights_blockwise_multi"
    with torch.cuda.device(dev):
        _check(name, getattr(_lib, name)(descs, len(ws), _stream(ws[0])))
    return res


def quantize_weights_blockwise_frag_multi(ws, outs=None):
    """quantize_weights_blockwise_multi with the codes in fragment order."""
    return quantize_weights_blockwise_multi(ws, outs, frag=True)


def quantize_act_per_token_group(x, out=None, scale=None):
    """BF16 activations [M, K] -> (E4M3 codes uint8 [M, K]; float32 scales [M, ceil(K/128)])."""
    if x.dim() != 2:
        raise ValueError("activations must be [M, K]")
    m, k = x.shape
    _require(x, "x", _BF16, x.shape)
    if out is None:
        out = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((m, _cdiv(k, BLOCK)), dtype=torch.float32, device=x.device)
    _require(out, "out", _U8, (m, k), x.device)
    _require(scale, "scale", torch.float32, (m, _cdiv(k, BLOCK)), x.device)
    with torch.cuda.device(x.device):
        _check("quantize_act_per_token_group",
               _lib.quantize_act_per_token_group(_ptr(x), _ptr(out), _ptr(scale), m, k, _stream(x)))
    return out, scale


def quantize_acts_per_token_group_multi(xs, outs=None, frag=False):
    """Several BF16 activations [M, K] (any shapes) in one launch -> list of
    (codes, scales), each exactly what quantize_act_per_token_group gives it
    (``frag``: what quantize_act_per_token_group_frag gives it, M % 16 == 0
    and K % 128 == 0).  ``outs``: optional list of (codes, scales) to fill."""
    xs = list(xs)
    if len(xs) > MAX_ACT_DESCS:
        raise ValueError(f"at most {MAX_ACT_DESCS} activations per call")
    if not xs:
        return []
    dev = xs[0].device
    res = []
    descs = (_ActDesc * len(xs))()
    for i, x in enumerate(xs):
        if x.dim() != 2:
            raise ValueError("each activation must be [M, K]")
        m, k = x.shape
        _require(x, f"x[{i}]", _BF16, (m, k), dev)
        if outs is None:
            q = torch.empty((m, k), dtype=torch.uint8, device=dev)
            s = torch.empty((m, _cdiv(k, BLOCK)), dtype=torch.float32, device=dev)
        else:
            q, s = outs[i]
        _require(q, f"out[{i}]", _U8, (m, k), dev)
        _require(s, f"scale[{i}]", torch.float32, (m, _cdiv(k, BLOCK)), dev)
        descs[i] = _ActDesc(_ptr(_u16(x)).value, _ptr(q).value, _ptr(s).value, m, k)
        res.append((q, s))
    name = "quantize_acts_per_token_group_frag_multi" if frag else "quantize_acts_per_token_group_multi"
    with torch.cuda.device(dev):
        _check(name, getattr(_lib, name)(descs, len(xs), _stream(xs[0])))
    return res


def quantize_acts_per_token_group_frag_multi(xs, outs=None):
    """quantize_acts_per_token_group_multi with codes in fragment order."""
    return quantize_acts_per_token_group_multi(xs, outs, frag=True)


def quantize_act_per_token_group_frag(x, out=None, scale=None):
    """BF16 activations [M, K] (M % 16 == 0, K % 128 == 0) -> (E4M3 codes uint8 [M, K] in the MFMA
    fragment order of gemm_w8a8_blockscaled_afrag; float32 scales [M, K/128])."""
    if x.dim() != 2:
        raise ValueError("activations must be [M, K]")
    m, k = x.shape
    if m % 16 or k % BLOCK:
        raise ValueError("fragment order needs M % 16 == 0 and K % 128 == 0")
    _require(x, "x", _BF16, x.shape)
    if out is None:
        out = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((m, k // BLOCK), dtype=torch.float32, device=x.device)
    _require(out, "out", _U8, (m, k), x.device)
    _require(scale, "scale", torch.float32, (m, k // BLOCK), x.device)
    with torch.cuda.device(x.device):
        _check("quantize_act_per_token_group_frag",
               _lib.quantize_act_per_token_group_frag(_ptr(x), _ptr(out), _ptr(scale), m, k, _stream(x)))
    return out, scale


def gemm_w8a8_blockscaled_afrag(a_frag, a_scale, w, w_scale, out=None, wfrag=False):
    """gemm_w8a8_blockscaled with the activation codes in fragment order (quantize_act_per_token_group_frag);
    M % 16 == 0 and K % 128 == 0.  ``wfrag``: the weight codes in fragment order too
    (gemm_w8a8_blockscaled_frag; N % 16 == 0)."""
    m, k = a_frag.shape
    n = w.shape[0]
    _require(a_frag, "a_frag", _U8, (m, k))
    dev = a_frag.device
    _require(a_scale, "a_scale", torch.float32, (m, k // BLOCK), dev)
    _require(w, "w", _U8, (n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (_cdiv(n, BLOCK), k // BLOCK), dev)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (m, n), dev)
    name = "gemm_w8a8_blockscaled_frag" if wfrag else "gemm_w8a8_blockscaled_afrag"
    with torch.cuda.device(dev):
        _check(name, getattr(_lib, name)(_ptr(a_frag), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(_u16(out)),
                                         m, n, k, _stream(a_frag)))
    return out


def gemm_w8a8_blockscaled_frag(a_frag, a_scale, w_frag, w_scale, out=None):
    """The GEMM with both operands' codes in fragment order (quantize_act_per_token_group_frag,
    quantize_weight_blockwise_frag); M % 16 == 0, N % 16 == 0, K % 128 == 0."""
    return gemm_w8a8_blockscaled_afrag(a_frag, a_scale, w_frag, w_scale, out, wfrag=True)


def gemm_w8a8_blockscaled(a, a_scale, w, w_scale, out=None, tile=None):
    """y[M, N] (bfloat16) = dequant(a) @ dequant(w).T with FP32 accumulation.

    ``tile`` (a name of TILES) runs that tile kernel instead of the library's
    choice (gemm_w8a8_blockscaled_tile)."""
    m, k = a.shape
    n = w.shape[0]
    _require(a, "a", _U8, (m, k))
    dev = a.device
    _require(a_scale, "a_scale", torch.float32, (m, k // BLOCK), dev)
    _require(w, "w", _U8, (n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (_cdiv(n, BLOCK), k // BLOCK), dev)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (m, n), dev)
    with torch.cuda.device(dev):
        if tile is None:
            _check("gemm_w8a8_blockscaled",
                   _lib.gemm_w8a8_blockscaled(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(_u16(out)), m, n,
                                              k, _stream(a)))
        else:
            _check("gemm_w8a8_blockscaled_tile",
                   _lib.gemm_w8a8_blockscaled_tile(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(_u16(out)), m,
                                                   n, k, _tile_id(tile), _stream(a)))
    return out


def splitk_workspace_bytes(m, n, k):
    """Workspace bytes gemm_w8a8_blockscaled_splitk needs for (M, N, K) on the current device (0: no split)."""
    b = ctypes.c_int64(0)
    _check("gemm_w8a8_blockscaled_splitk_workspace",
           _lib.gemm_w8a8_blockscaled_splitk_workspace(int(m), int(n), int(k), ctypes.byref(b)))
    return b.value


def gemm_w8a8_blockscaled_splitk(a, a_scale, w, w_scale, out=None, workspace=None):
    """gemm_w8a8_blockscaled for few activation rows (M <= 256) with K split
    over more workgroups; ``workspace``: a uint8 device tensor of at least
    splitk_workspace_bytes(M, N, K) bytes (allocated here when None)."""
    m, k = a.shape
    n = w.shape[0]
    _require(a, "a", _U8, (m, k))
    dev = a.device
    _require(a_scale, "a_scale", torch.float32, (m, k // BLOCK), dev)
    _require(w, "w", _U8, (n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (_cdiv(n, BLOCK), k // BLOCK), dev)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (m, n), dev)
    with torch.cuda.device(dev):
        if workspace is None:
            need = splitk_workspace_bytes(m, n, k)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of a")
        _check("gemm_w8a8_blockscaled_splitk",
               _lib.gemm_w8a8_blockscaled_splitk(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(_u16(out)), m,
                                                 n, k, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream(a)))
    return out


def gemm_w8a8_blockscaled_splitk_noalloc(a, a_scale, w, w_scale, out):
    """gemm_w8a8_blockscaled_splitk with the library's static scratch instead
    of a workspace (for callers that cannot allocate: ``out`` must be given;
    nothing is allocated here either)."""
    m, k = a.shape
    n = w.shape[0]
    _require(a, "a", _U8, (m, k))
    dev = a.device
    _require(a_scale, "a_scale", torch.float32, (m, k // BLOCK), dev)
    _require(w, "w", _U8, (n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (_cdiv(n, BLOCK), k // BLOCK), dev)
    _require(out, "out", _BF16, (m, n), dev)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    with torch.cuda.device(dev):
        _check("gemm_w8a8_blockscaled_splitk_noalloc",
               _lib.gemm_w8a8_blockscaled_splitk_noalloc(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale),
                                                         _ptr(_u16(out)), m, n, k, _stream(a)))
    return out


def grouped_gemm_w8a8_blockscaled(a, a_scale, w, w_scale, group_offsets, out=None, tile=None):
    """Rows [off[e], off[e+1]) of a use expert e's weights w[e]; returns bfloat16 [M_total, N].
    ``tile``: a grouped tile kernel of TILES (grouped_gemm_w8a8_blockscaled_tile)."""
    m, k = a.shape
    g, n, _ = w.shape
    _require(a, "a", _U8, (m, k))
    dev = a.device
    _require(a_scale, "a_scale", torch.float32, (m, k // BLOCK), dev)
    _require(w, "w", _U8, (g, n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (g, _cdiv(n, BLOCK), k // BLOCK), dev)
    _require(group_offsets, "group_offsets", torch.int32, (g + 1,), dev)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (m, n), dev)
    with torch.cuda.device(dev):
        if tile is None:
            _check("grouped_gemm_w8a8_blockscaled",
                   _lib.grouped_gemm_w8a8_blockscaled(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale),
                                                      _ptr(group_offsets), _ptr(_u16(out)), m, n, k, g, _stream(a)))
        else:
            _check("grouped_gemm_w8a8_blockscaled_tile",
                   _lib.grouped_gemm_w8a8_blockscaled_tile(_ptr(a), _ptr(a_scale), m, None, 1, _ptr(w), _ptr(w_scale),
                                                           _ptr(group_offsets), _ptr(_u16(out)), m, n, k, g,
                                                           _tile_id(tile), _stream(a)))
    return out


def grouped_gemm_w8a8_blockscaled_gather(a, a_scale, a_rows, a_row_div, w, w_scale, group_offsets, out=None,
                                         tile=None):
    """Output row m uses row a_rows[m] // a_row_div of a [M_a, K] and expert e's
    weights for m in [off[e], off[e+1]); returns bfloat16 [len(a_rows), N].
    ``tile``: a grouped tile kernel of TILES (grouped_gemm_w8a8_blockscaled_tile)."""
    m_a, k = a.shape
    g, n, _ = w.shape
    _require(a, "a", _U8, (m_a, k))
    dev = a.device
    m = a_rows.numel()
    _require(a_scale, "a_scale", torch.float32, (m_a, k // BLOCK), dev)
    _require(a_rows, "a_rows", torch.int32, (m,), dev)
    _require(w, "w", _U8, (g, n, k), dev)
    _require(w_scale, "w_scale", torch.float32, (g, _cdiv(n, BLOCK), k // BLOCK), dev)
    _require(group_offsets, "group_offsets", torch.int32, (g + 1,), dev)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (m, n), dev)
    with torch.cuda.device(dev):
        if tile is None:
            _check("grouped_gemm_w8a8_blockscaled_gather",
                   _lib.grouped_gemm_w8a8_blockscaled_gather(_ptr(a), _ptr(a_scale), m_a, _ptr(a_rows),
                                                             int(a_row_div), _ptr(w), _ptr(w_scale),
                                                             _ptr(group_offsets), _ptr(_u16(out)), m, n, k, g,
                                                             _stream(a)))
        else:
            _check("grouped_gemm_w8a8_blockscaled_tile",
                   _lib.grouped_gemm_w8a8_blockscaled_tile(_ptr(a), _ptr(a_scale), m_a, _ptr(a_rows), int(a_row_div),
                                                           _ptr(w), _ptr(w_scale), _ptr(group_offsets),
                                                           _ptr(_u16(out)), m, n, k, g, _tile_id(tile), _stream(a)))
    return out


def check_group_offsets(group_offsets, m_total):
    """Host check of the grouped GEMMs' offsets contract (int32 [G+1] on the
    device: [0] = 0, non-decreasing, [G] = M_total); raises FP8BQError if it
    is broken.  Synchronous."""
    g = group_offsets.numel() - 1
    _require(group_offsets, "group_offsets", torch.int32, (g + 1,))
    with torch.cuda.device(group_offsets.device):
        _check("fp8bq_check_group_offsets",
               _lib.fp8bq_check_group_offsets(_ptr(group_offsets), g, int(m_total), _stream(group_offsets)))


def encode_e4m3(v, method=1, out=None):
    """float32 [n] -> E4M3 codes uint8 [n] with the library's conversion (see fp8bq.h for methods)."""
    if v.dim() != 1:
        raise ValueError("encode_e4m3 takes a 1-D tensor")
    _require(v, "v", torch.float32, v.shape)
    if out is None:
        out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _require(out, "out", torch.uint8, v.shape, v.device)
    with torch.cuda.device(v.device):
        _check("fp8bq_encode_e4m3", _lib.fp8bq_encode_e4m3(_ptr(v), _ptr(out), v.numel(), int(method), _stream(v)))
    return out


_IW_MODES = {"tis": 0, "mis": 1}


def token_importance_weights(logp_train, logp_rollout, C=2.0, mode="tis", mask=None, advantages=None,
                             out=None, out_adv=None):
    """Per-token rollout-correction weights w = exp(logp_train - logp_rollout).

    ``mode="tis"`` limits w to [1/C, C]; ``mode="mis"`` sets w = 0 outside
    that band.  float32 log-probabilities of any one shape (e.g. [responses,
    max_len]); ``mask`` (bool / uint8, same shape, 0 = padding) zeroes
    padding; with ``advantages`` the call also returns w * A.  Returns ``w``
    or ``(w, w * A)``.
    """
    if mode not in _IW_MODES:
        raise ValueError(f"mode must be one of {sorted(_IW_MODES)}")
    shape = tuple(logp_train.shape)
    _require(logp_train, "logp_train", torch.float32, shape)
    dev = logp_train.device
    _require(logp_rollout, "logp_rollout", torch.float32, shape, dev)
    if mask is not None:
        _require(mask, "mask", (torch.bool, torch.uint8), shape, dev)
        mask = mask.view(torch.uint8)
    if advantages is not None:
        _require(advantages, "advantages", torch.float32, shape, dev)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, shape, dev)
    if advantages is not None:
        if out_adv is None:
            out_adv = torch.empty(shape, dtype=torch.float32, device=dev)
        _require(out_adv, "out_adv", torch.float32, shape, dev)
    elif out_adv is not None:
        raise ValueError("out_adv given without advantages")
    with torch.cuda.device(dev):
        _check("token_importance_weights",
               _lib.token_importance_weights(_ptr(logp_train), _ptr(logp_rollout), _ptr(mask), _ptr(advantages),
                                             _ptr(out), _ptr(out_adv), logp_train.numel(), float(C),
                                             _IW_MODES[mode], _stream(logp_train)))
    return out if advantages is None else (out, out_adv)


def moe_sort_by_expert(topk_ids, num_experts, offsets=None, sorted_pair=None, pair_row=None):
    """Routing ids int32 [T, k] -> (group_offsets int32 [E+1], sorted_pair int32 [T*k], pair_row int32 [T*k])."""
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [tokens, k]")
    T, k = topk_ids.shape
    dev = topk_ids.device
    _require(topk_ids, "topk_ids", torch.int32, (T, k))
    E = int(num_experts)
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if sorted_pair is None:
        sorted_pair = torch.empty(T * k, dtype=torch.int32, device=dev)
    if pair_row is None:
        pair_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    _require(offsets, "offsets", torch.int32, (E + 1,), dev)
    _require(sorted_pair, "sorted_pair", torch.int32, (T * k,), dev)
    _require(pair_row, "pair_row", torch.int32, (T * k,), dev)
    with torch.cuda.device(dev):
        _check("moe_sort_by_expert", _lib.moe_sort_by_expert(_ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(sorted_pair),
                                                             _ptr(pair_row), _stream(topk_ids)))
    return offsets, sorted_pair, pair_row


def moe_gather_quantize_act(x, sorted_pair, k, out=None, scale=None):
    """BF16 x [T, K] and sorted pairs [R] -> (E4M3 rows [R, K] of tokens sorted_pair // k, scales [R, K/128])."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, K]")
    T, K = x.shape
    dev = x.device
    _require(x, "x", _BF16, (T, K))
    R = sorted_pair.numel()
    _require(sorted_pair, "sorted_pair", torch.int32, (R,), dev)
    if out is None:
        out = torch.empty((R, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((R, K // BLOCK), dtype=torch.float32, device=dev)
    _require(out, "out", _U8, (R, K), dev)
    _require(scale, "scale", torch.float32, (R, K // BLOCK), dev)
    with torch.cuda.device(dev):
        _check("moe_gather_quantize_act",
               _lib.moe_gather_quantize_act(_ptr(_u16(x)), _ptr(sorted_pair), R, T, int(k), K, _ptr(out), _ptr(scale),
                                            _stream(x)))
    return out, scale


def silu_mul_quantize_act(y, out=None, scale=None, h_out=None):
    """fc1 output BF16 [M, 2F] = [gate | up] -> (E4M3 codes of BF16(SiLU(gate) * up) [M, F], scales [M, F/128]).

    With ``h_out`` (BF16 [M, F]) the BF16 h is stored as well."""
    if y.dim() != 2 or y.shape[1] % 2:
        raise ValueError("y must be [rows, 2F]")
    M, F = y.shape[0], y.shape[1] // 2
    dev = y.device
    _require(y, "y", _BF16, (M, 2 * F))
    if out is None:
        out = torch.empty((M, F), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((M, _cdiv(F, BLOCK)), dtype=torch.float32, device=dev)
    _require(out, "out", _U8, (M, F), dev)
    _require(scale, "scale", torch.float32, (M, _cdiv(F, BLOCK)), dev)
    if h_out is not None:
        _require(h_out, "h_out", _BF16, (M, F), dev)
    with torch.cuda.device(dev):
        _check("silu_mul_quantize_act",
               _lib.silu_mul_quantize_act(_ptr(_u16(y)), M, F, _ptr(out), _ptr(scale),
                                          _ptr(None if h_out is None else _u16(h_out)), _stream(y)))
    return out, scale


def moe_combine(y, pair_row, topk_weights, out=None):
    """fc2 output BF16 [M, H], pair_row [T*k], weights float32 [T, k] -> BF16 [T, H] weighted sums."""
    if y.dim() != 2 or topk_weights.dim() != 2:
        raise ValueError("y must be [rows, H] and topk_weights [tokens, k]")
    M, H = y.shape
    T, k = topk_weights.shape
    dev = y.device
    _require(y, "y", _BF16, (M, H))
    _require(pair_row, "pair_row", torch.int32, (T * k,), dev)
    _require(topk_weights, "topk_weights", torch.float32, (T, k), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require(out, "out", _BF16, (T, H), dev)
    with torch.cuda.device(dev):
        _check("moe_combine", _lib.moe_combine(_ptr(_u16(y)), _ptr(pair_row), _ptr(topk_weights), T, k, H, M,
                                               _ptr(_u16(out)), _stream(y)))
    return out


def grouped_gemm_w8a8_blockscaled_gather_silu(a, a_scale, a_rows, a_row_div, w, w_scale, group_offsets, h=None,
                                              h_scale=None):
    """MoE fc1 with SiLU(gate) * up quantized in its epilogue: w E4M3 [G, 2F, K] ([gate; up]),
    rows gathered as in grouped_gemm_w8a8_blockscaled_gather -> (h codes uint8 [len(a_rows), F],
    float32 scales [len(a_rows), F/128]), exactly those of silu_mul_quantize_act of the BF16 fc1 output."""
    m_a, k = a.shape
    g, n2, _ = w.shape
    f = n2 // 2
    dev = a.device
    m = a_rows.numel()
    _require(a, "a", _U8, (m_a, k))
    _require(a_scale, "a_scale", torch.float32, (m_a, k // BLOCK), dev)
    _require(a_rows, "a_rows", torch.int32, (m,), dev)
    _require(w, "w", _U8, (g, n2, k), dev)
    _require(w_scale, "w_scale", torch.float32, (g, _cdiv(n2, BLOCK), k // BLOCK), dev)
    _require(group_offsets, "group_offsets", torch.int32, (g + 1,), dev)
    if n2 % 2:
        raise ValueError("w must hold [gate; up] rows (an even count)")
    if h is None:
        h = torch.empty((m, f), dtype=torch.uint8, device=dev)
    if h_scale is None:
        h_scale = torch.empty((m, _cdiv(f, BLOCK)), dtype=torch.float32, device=dev)
    _require(h, "h", _U8, (m, f), dev)
    _require(h_scale, "h_scale", torch.float32, (m, _cdiv(f, BLOCK)), dev)
    with torch.cuda.device(dev):
        _check("grouped_gemm_w8a8_blockscaled_gather_silu",
               _lib.grouped_gemm_w8a8_blockscaled_gather_silu(_ptr(a), _ptr(a_scale), m_a, _ptr(a_rows), int(a_row_div),
                                                              _ptr(w), _ptr(w_scale), _ptr(group_offsets), _ptr(h),
                                                              _ptr(h_scale), m, f, k, g, _stream(a)))
    return h, h_scale


def moe_expert_ffn(x, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, fused=True):
    """One MoE expert FFN layer through the library's kernels only.

    x BF16 [T, H]; topk_ids int32 [T, k]; topk_weights float32 [T, k];
    w1 E4M3 [E, 2F, H] (fc1 = [gate; up]) with scales [E, 2F/128, H/128];
    w2 E4M3 [E, H, F] (fc2) with scales [E, H/128, F/128].  Returns BF16 [T, H].
    ``fused``: fc1 with the SiLU * up quantization in its epilogue (same
    result bits as the separate kernels).
    """
    E, H = w1.shape[0], x.shape[1]
    k = topk_ids.shape[1]
    offsets, sorted_pair, pair_row = moe_sort_by_expert(topk_ids, E)
    a, a_s = quantize_act_per_token_group(x)   # once per token; fc1 gathers the rows
    if fused:
        h, h_s = grouped_gemm_w8a8_blockscaled_gather_silu(a, a_s, sorted_pair, k, w1, w1_scale, offsets)
    else:
        y1 = grouped_gemm_w8a8_blockscaled_gather(a, a_s, sorted_pair, k, w1, w1_scale, offsets)
        h, h_s = silu_mul_quantize_act(y1)
    y2 = grouped_gemm_w8a8_blockscaled(h, h_s, w2, w2_scale, offsets)
    return moe_combine(y2, pair_row, topk_weights)


def kv_scale_calibrate(k, v=None, per_head=True, k_scale=None, v_scale=None):
    """K (and V) BF16 [T, H, D] of a rollout's first forward -> float32 scales
    [H] (per_head) or [1]: s = fl32(max |x| / 448).  Returns (k_scale, v_scale)."""
    if k.dim() != 3:
        raise ValueError("k must be [tokens, heads, head_dim]")
    T, H, D = k.shape
    dev = k.device
    _require(k, "k", _BF16, (T, H, D))
    if v is not None:
        _require(v, "v", _BF16, (T, H, D), dev)
    n = H if per_head else 1
    if k_scale is None:
        k_scale = torch.empty(n, dtype=torch.float32, device=dev)
    _require(k_scale, "k_scale", torch.float32, (n,), dev)
    if v is not None:
        if v_scale is None:
            v_scale = torch.empty(n, dtype=torch.float32, device=dev)
        _require(v_scale, "v_scale", torch.float32, (n,), dev)
    else:
        v_scale = None
    with torch.cuda.device(dev):
        _check("kv_scale_calibrate",
               _lib.kv_scale_calibrate(_ptr(_u16(k)), _ptr(None if v is None else _u16(v)), T, H, D, int(bool(per_head)),
                                       _ptr(k_scale), _ptr(v_scale), _stream(k)))
    return k_scale, v_scale


def kv_cache_write_fp8(k, v, slot_mapping, k_scale, v_scale, k_cache, v_cache=None):
    """Quantize K (and V) BF16 [T, H, D] with fixed scales and store token t in
    slot slot_mapping[t] (int32 [T]; out of range = padding) of the E4M3
    caches [S, H, D] (uint8).  Per-head scales have H entries, per-layer 1."""
    T, H, D = k.shape
    dev = k.device
    _require(k, "k", _BF16, (T, H, D))
    _require(slot_mapping, "slot_mapping", torch.int32, (T,), dev)
    n = k_scale.numel()
    if n not in (1, H):
        raise ValueError("k_scale must have 1 or H entries")
    per_head = n == H and H > 1
    _require(k_scale, "k_scale", torch.float32, (n,), dev)
    S = k_cache.shape[0]
    _require(k_cache, "k_cache", _U8, (S, H, D), dev)
    if v is not None:
        _require(v, "v", _BF16, (T, H, D), dev)
        _require(v_scale, "v_scale", torch.float32, (n,), dev)
        _require(v_cache, "v_cache", _U8, (S, H, D), dev)
    with torch.cuda.device(dev):
        _check("kv_cache_write_fp8",
               _lib.kv_cache_write_fp8(_ptr(_u16(k)), _ptr(None if v is None else _u16(v)), _ptr(slot_mapping),
                                       _ptr(k_scale), _ptr(None if v is None else v_scale), int(per_head),
                                       _ptr(k_cache), _ptr(None if v is None else v_cache), T, H, D, S, _stream(k)))
    return k_cache, v_cache


def quantize_weight_blockwise_dual(w, forward=True):
    """BF16 W [N, K] or [B, N, K] -> ((W codes, scales) or (None, None), (W^T codes [.., K, N], scales))."""
    batched = w.dim() == 3
    wb = w if batched else w.unsqueeze(0)
    b, n, k = wb.shape
    _require(wb, "w", _BF16, (b, n, k))
    dev = w.device
    nb, kb = _cdiv(n, BLOCK), _cdiv(k, BLOCK)
    q = torch.empty((b, n, k), dtype=torch.uint8, device=dev) if forward else None
    s = torch.empty((b, nb, kb), dtype=torch.float32, device=dev) if forward else None
    qt = torch.empty((b, k, n), dtype=torch.uint8, device=dev)
    st = torch.empty((b, kb, nb), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("quantize_weight_blockwise_dual",
               _lib.quantize_weight_blockwise_dual(_ptr(_u16(wb)), _ptr(q), _ptr(s), _ptr(qt), _ptr(st), b, n, k,
                                                   _stream(w)))
    sq = (lambda t: t) if batched else (lambda t: None if t is None else t[0])
    return (sq(q), sq(s)), (sq(qt), sq(st))


def quantize_act_dual(x, forward=True):
    """BF16 x [M, K] -> ((codes [M, K], scales [M, K/128]) or (None, None),
    (x^T codes [K, M], scales [K, ceil(M/128)]) in groups along the tokens)."""
    m, k = x.shape
    _require(x, "x", _BF16, (m, k))
    dev = x.device
    q = torch.empty((m, k), dtype=torch.uint8, device=dev) if forward else None
    s = torch.empty((m, _cdiv(k, BLOCK)), dtype=torch.float32, device=dev) if forward else None
    qt = torch.empty((k, m), dtype=torch.uint8, device=dev)
    st = torch.empty((k, _cdiv(m, BLOCK)), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("quantize_act_dual",
               _lib.quantize_act_dual(_ptr(_u16(x)), _ptr(q), _ptr(s), _ptr(qt), _ptr(st), m, k, _stream(x)))
    return (q, s), (qt, st)


def raw_library():
    """The ctypes handle, for callers that marshal pointers themselves."""
    return _lib
