"""Shared helpers for the GPU parity tests: seeded inputs, the library layer, tolerances."""
from __future__ import annotations

import functools
import sys

import numpy as np

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

# Parity bar on bf16 outputs: max-abs-err <= 2e-2 and relative L2 <= 1e-2.
MAX_ABS = 2e-2
REL_L2 = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(gpu: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = gpu - ref
    return float(np.max(np.abs(err))), float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))


def assert_close(gpu, ref, what: str, max_abs: float = MAX_ABS, rel_l2: float = REL_L2):
    ma, rl = metrics(gpu, ref)
    log(f"  {what}: max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}"


@functools.lru_cache(maxsize=1)
def weights():
    bits = synth.make_weights_bf16(seed=0)
    w64 = {k: synth.bf16_bits_to_f64(v) for k, v in bits.items()}
    return bits, w64


@functools.lru_cache(maxsize=2)
def layer(max_positions: int = 16384):
    bits, _ = weights()
    return binding.Layer(binding.weights_to_device(bits), max_positions=max_positions)


def y_of(t) -> np.ndarray:
    return synth.bf16_bits_to_f64(binding.tensor_to_bf16_bits(t))


def entries_f64(entry_bytes_rows) -> tuple[np.ndarray, np.ndarray]:
    """bf16 cache slots ([n, 1152] uint8, cpu numpy) -> (c_hat [n,512], k_pe [n,64]) float64."""
    bits = np.ascontiguousarray(entry_bytes_rows).view(np.uint16).reshape(-1, 576)
    v = synth.bf16_bits_to_f64(bits)
    return v[:, :512], v[:, 512:]


def oracle_cfg() -> omla.Config:
    return omla.KIMI_K2
