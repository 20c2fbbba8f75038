"""FP8 (OCP E4M3FN) arithmetic for the oracle. TEST INFRASTRUCTURE ONLY.

Source: "Key-value latent" page, linear excerpt (config.json quantization_config): weights in
e4m3 with one scale per 128 x 128 block, "dynamic" activations. The pages give the format
name and block size only; the activation scheme below is the reading stated in the package
docstring (per token, per aligned group of 128 inputs, scale = fl32(amax / 448)).

E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is subnormal
(m/8 * 2^-6); 0x7F/0xFF are NaN; there is no infinity; the largest finite value is 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GROUP = 128


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN codes (uint8) to float64 from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_POS_VALUES = e4m3_value(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to the even code, saturating at +-448.

    Exact: the distances are formed in float64 from values with at most 24 significant bits.
    A negative input that rounds to zero gives code 0x80 (negative zero).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_POS_VALUES[hi] == a, hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_1x128(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic activation quantiser: per row, per aligned group of 128 features.

    The activation is taken in float32 (a32 = fl32(a)). For each group:
    s = fl32(amax / 448) with amax = max |a32| (s = 1 when amax is 0), and
    code = e4m3(fl32(a32 / s)) with round-to-nearest-even and saturation.
    Returns codes [..., K] (uint8) and scales [..., K/128] (float32).
    """
    a32 = np.asarray(a).astype(np.float32)
    k = a32.shape[-1]
    if k % GROUP:
        raise ValueError("feature count must be a multiple of 128")
    g = a32.reshape(a32.shape[:-1] + (k // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = (g / s[..., None]).astype(np.float32)
    codes = e4m3_encode(q).reshape(a32.shape)
    return codes, s


def dequant_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code value * group scale, exact in float64."""
    v = e4m3_value(codes)
    k = v.shape[-1]
    g = v.reshape(v.shape[:-1] + (k // GROUP, GROUP))
    return (g * np.asarray(scales, dtype=np.float64)[..., None]).reshape(v.shape)


def fake_quant_1x128(a: np.ndarray) -> np.ndarray:
    """The value a projection sees after dynamic quantisation: dequant(quantize(a))."""
    codes, s = quantize_1x128(a)
    return dequant_1x128(codes, s)


def dequant_weight(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Block-scaled weight [out, in]: code value * scale[o // 128, i // 128] (exact in float64).

    The scale grid is [ceil(out/128), ceil(in/128)]; a ragged last block row (kv_a: 576 rows =
    4 full blocks + 64 rows) uses its own scale.
    """
    v = e4m3_value(codes)
    n, k = v.shape
    s = np.asarray(scales, dtype=np.float64)
    if s.shape != (-(-n // block), -(-k // block)):
        raise ValueError(f"scale grid {s.shape} does not match weight {v.shape}")
    s_full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:n, :k]
    return v * s_full
