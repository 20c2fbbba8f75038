"""Seeded synthetic inputs for the MLA layer: weights, hidden states, cache lengths.

This module generates data only. It holds none of the layer's arithmetic: no
projection, normalisation, rotation, attention or quantisation of activations
lives here. Both the float64 CPU oracle (through the tests and the bench) and
the HIP path are fed from it, so they see the same input bits.

Shapes and distributions follow the Kimi-K2 configuration printed on the
"KV cache" page (config.json excerpt: hidden_size 7168, q_lora_rank 1536,
kv_lora_rank 512, 64 heads, qk_nope_head_dim 128, qk_rope_head_dim 64,
v_head_dim 128, initializer_range 0.02, torch_dtype bfloat16) and the FP8
block format on the "Key-value latent" page (quantization_config: e4m3,
weight_block_size [128, 128]).

Representation:
  * bf16 tensors are numpy uint16 arrays holding the bfloat16 bit patterns.
  * FP8 weights are numpy uint8 arrays of OCP E4M3FN codes plus a float32
    scale grid of shape [ceil(out/128), ceil(in/128)].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    """Layer dimensions (defaults: Kimi-K2, from the config on the "KV cache" page)."""

    hidden: int = 7168
    q_lora: int = 1536
    kv_lora: int = 512
    heads: int = 64
    nope: int = 128
    rope: int = 64
    v: int = 128

    @property
    def qk(self) -> int:
        return self.nope + self.rope

    @property
    def entry(self) -> int:
        """Features held per cached position in the latent layout (512 + 64)."""
        return self.kv_lora + self.rope


KIMI_K2 = Dims()

# Weight names in generation order. Each entry: (name, out, in) or (name, n) for gains.
def weight_shapes(d: Dims = KIMI_K2) -> list[tuple[str, tuple[int, ...]]]:
    return [
        ("q_a", (d.q_lora, d.hidden)),
        ("q_a_norm", (d.q_lora,)),
        ("q_b", (d.heads * d.qk, d.q_lora)),
        ("kv_a", (d.kv_lora + d.rope, d.hidden)),
        ("kv_a_norm", (d.kv_lora,)),
        ("kv_b", (d.heads * (d.nope + d.v), d.kv_lora)),
        ("o", (d.hidden, d.heads * d.v)),
    ]


PROJECTIONS = ("q_a", "q_b", "kv_a", "kv_b", "o")
GAINS = ("q_a_norm", "kv_a_norm")


# ----------------------------------------------------------------------------------------------
# bf16 bit handling (data representation only)
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite (normal draws), so NaN handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------------------------
def _normal_bf16(rng: np.random.Generator, shape, mean: float, std: float) -> np.ndarray:
    v = rng.normal(mean, std, size=shape)  # float64 draw
    return f32_to_bf16_bits(v.astype(np.float32))


def make_weights_bf16(d: Dims = KIMI_K2, seed: int = 0, std: float = 0.02, gain_std: float = 0.1,
                      zero: tuple[str, ...] = ()) -> dict[str, np.ndarray]:
    """bf16 weights, [out, in] row-major: projections N(0, std), RMSNorm gains 1 + N(0, gain_std).

    Drawn from one PCG64 stream in the fixed order of `weight_shapes`. Names listed in `zero`
    are replaced by zeros after drawing (the stream is unchanged).
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in weight_shapes(d):
        if name in GAINS:
            out[name] = _normal_bf16(rng, shape, 1.0, gain_std)
        else:
            out[name] = _normal_bf16(rng, shape, 0.0, std)
        if name in zero:
            out[name] = np.zeros_like(out[name])
    return out


def e4m3_encode_sat(v: np.ndarray) -> np.ndarray:
    """float -> OCP E4M3FN codes, round to nearest even, saturating to +-448 (weight generation only).

    Uses torch's CPU cast, which rounds to nearest even but does not saturate, so values are
    clamped to the finite range first.
    """
    import torch

    c = np.clip(np.asarray(v, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_weights_fp8(d: Dims = KIMI_K2, seed: int = 0, std: float = 0.02, gain_std: float = 0.1,
                     log2_lo: float = -10.0, log2_hi: float = -4.0) -> dict[str, np.ndarray]:
    """FP8 weights: per 128x128 block s = fl32(2^U(log2_lo, log2_hi)), code = e4m3(N(0,std)/s).

    Returns codes under each projection name, the float32 scale grid under "<name>_s" and bf16
    gains as in `make_weights_bf16`. Dequantised weights are about N(0, std).
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in weight_shapes(d):
        if name in GAINS:
            out[name] = _normal_bf16(rng, shape, 1.0, gain_std)
            continue
        n, k = shape
        nb, kb = -(-n // 128), -(-k // 128)
        s = np.exp2(rng.uniform(log2_lo, log2_hi, size=(nb, kb))).astype(np.float32)
        w = rng.normal(0.0, std, size=shape)
        s_full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:n, :k].astype(np.float64)
        out[name] = e4m3_encode_sat((w / s_full).astype(np.float32))
        out[name + "_s"] = s
    return out


def make_hidden(n_tokens: int, d: Dims = KIMI_K2, seed: int = 1000, std: float = 1.0) -> np.ndarray:
    """hidden_states [n_tokens, hidden] ~ N(0, std) in bf16 bits."""
    rng = np.random.default_rng(seed)
    return _normal_bf16(rng, (n_tokens, d.hidden), 0.0, std)


def make_block_norm(d: Dims = KIMI_K2, seed: int = 7, gain_std: float = 0.1) -> np.ndarray:
    """Decoder-block input RMSNorm gain [hidden] ~ 1 + N(0, gain_std) in bf16 bits."""
    rng = np.random.default_rng(seed)
    return _normal_bf16(rng, (d.hidden,), 1.0, gain_std)


def make_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-sequence cached lengths, uniform integers in [lo, hi] inclusive."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def packed_offsets(caps: np.ndarray, align: int = 16) -> tuple[np.ndarray, np.ndarray, int]:
    """Packed slot layout: capacity rounded up to `align`, offsets are the exclusive prefix sum."""
    caps = ((np.asarray(caps, dtype=np.int64) + align - 1) // align) * align
    offs = np.zeros_like(caps)
    if caps.size > 1:
        offs[1:] = np.cumsum(caps)[:-1]
    return offs, caps.astype(np.int32), int(caps.sum())


def make_cache_entries(n: int, d: Dims = KIMI_K2, seed: int = 2000, latent_std: float = 1.0,
                       kpe_std: float = 1.7) -> np.ndarray:
    """Synthetic latent cache entries [n, kv_lora + rope] in bf16 bits.

    The latent part stands for RMSNorm outputs (unit RMS times gains near 1: N(0, latent_std));
    the rotary part for the shared key of a 7168-wide N(0,1) input through N(0, 0.02) weights
    (std sqrt(7168) * 0.02 = 1.7; a rotation keeps it). Used where filling a long cache through
    the kv path would cost more than the test itself.
    """
    rng = np.random.default_rng(seed)
    lat = rng.normal(0.0, latent_std, size=(n, d.kv_lora))
    kpe = rng.normal(0.0, kpe_std, size=(n, d.rope))
    return f32_to_bf16_bits(np.concatenate([lat, kpe], axis=1).astype(np.float32))


def make_cache_entries_fp8(n: int, seed: int = 2100) -> np.ndarray:
    """Synthetic 784-byte FP8 cache slots [n, 784] (uint8) for timing long caches: 512 random
    E4M3FN codes (any finite code, either sign), four float32 group scales 2^U(-9, -6) and a
    float32 rotary key N(0, 1.7)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, size=(n, 512), dtype=np.uint8) | (rng.integers(0, 2, size=(n, 512), dtype=np.uint8) << 7)
    scales = np.exp2(rng.uniform(-9.0, -6.0, size=(n, 4))).astype(np.float32)
    kpe = rng.normal(0.0, 1.7, size=(n, 64)).astype(np.float32)
    out = np.empty((n, 784), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:528] = scales.view(np.uint8).reshape(n, 16)
    out[:, 528:] = kpe.view(np.uint8).reshape(n, 256)
    return out


def make_activations(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """A [rows, cols] N(0, std) activation matrix in bf16 bits (e.g. an o_proj input)."""
    rng = np.random.default_rng(seed)
    return _normal_bf16(rng, (rows, cols), 0.0, std)
