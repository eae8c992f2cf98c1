"""FP8 KV cache: per-step scale recalibration and the quantizing cache write.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.4 "KV-Cache Quantization"):

* "The Dynamic QKV Scale Recalibration Challenge", Paradigm 1: at the start
  of every rollout the engine observes the key and value tensors of the
  first forward pass under the new weights and derives per-layer or per-head
  FP8 scaling factors from them, then keeps them for the rest of the
  rollout.  ``kv_calibrate`` computes those factors for one layer.
* The cache stores K and V as 1-byte E4M3 values (half the BF16 footprint).
  ``kv_quantize`` / ``kv_cache_write`` quantize each token's K or V with the
  layer's fixed scales and store it in the token's cache slot.

Readings of what the pages leave open:

* The scale follows the same rule as the linear layers' blocks (§3.4.1: the
  largest magnitude maps to the E4M3 maximum): s = fl32(amax / 448), with
  amax over all calibration tokens of the layer (per-layer) or of one KV
  head (per-head).  K and V have separate scales.
* Quantized value: E4M3(fl32(x / s)), round to nearest even.  Later tokens
  may exceed the calibrated amax: their quotients saturate to +-448.  A
  zero scale (an all-zero calibration) gives +-448 for non-zero values and
  the signed zero for zeros (x / 0 = +-inf saturates; 0 / 0 is read as 0).
* Layout: K / V of T tokens as [T][H][D] BF16 (H KV heads of D elements);
  the cache as [S][H][D] E4M3 slots; token t goes to slot slot_mapping[t],
  and tokens whose slot is outside [0, S) (padding) are not written.

Pinned in ``tests/test_oracle_kv.py``.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32
from .e4m3 import E4M3_MAX, encode_e4m3
from .quant import quantize_tiles


def kv_calibrate(kv_bits, per_head):
    """Scales of one layer's K (or V) [T][H][D] BF16 bits: float32 [H] or [1]."""
    x = np.asarray(kv_bits, dtype=np.uint16)
    T, H, D = x.shape
    if per_head:
        tiles = x.transpose(1, 0, 2).reshape(H, T * D)       # one tile per head
    else:
        tiles = x.reshape(1, T * H * D)                      # one tile per layer
    _, scales = quantize_tiles(bf16_bits_to_f32(tiles))
    return scales


def kv_quantize(kv_bits, scales, per_head):
    """E4M3 codes [T][H][D] of K (or V) with fixed scales ([H] or [1])."""
    x = bf16_bits_to_f32(np.asarray(kv_bits, dtype=np.uint16))
    s = np.asarray(scales, dtype=np.float32)
    T, H, D = x.shape
    sb = (s[None, :, None] if per_head else np.full((1, 1, 1), s[0], np.float32))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = x / sb                                           # float32 IEEE quotient
    q = np.where(np.isnan(q), np.copysign(np.float32(0.0), x), q)   # 0 / 0: signed zero
    q = np.clip(q, -2 * E4M3_MAX, 2 * E4M3_MAX)              # beyond the range: saturates below
    return encode_e4m3(q.astype(np.float32))


def kv_cache_write(cache, kv_bits, scales, per_head, slot_mapping):
    """Copy of cache [S][H][D] with each token's codes in its slot."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    codes = kv_quantize(kv_bits, scales, per_head)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    ok = (slots >= 0) & (slots < out.shape[0])
    out[slots[ok]] = codes[ok]
    return out
