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


def bf16_unit(ref: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |ref| (2^(e-7) for 2^e <= |ref| < 2^(e+1); 8 significant
    bits). Zero maps to the smallest normal spacing."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def assert_bf16_rounding_of(gpu, ref, what: str, rel_floor: float = 1e-4):
    """A bf16 value the GPU rounded from a float32 computation of an exact oracle value: within
    one bf16 unit of the oracle (half a unit for the rounding, the rest for the float32 sums),
    plus rel_floor of the largest |ref| for elements so close to zero that float32 summation
    error exceeds their own bf16 spacing."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = bf16_unit(ref) + rel_floor * float(np.max(np.abs(ref)))
    worst = float(np.max(err / bound))
    log(f"  {what}: max |err| / (1 bf16 unit + floor) = {worst:.3f}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert worst <= 1.0, f"{what}: an element is more than one bf16 unit from the oracle ({worst:.3f})"


def assert_close_carried(gpu, ref, carried, what: str):
    """A later layer of a stack: its bf16 output against the oracle's unrounded value, where the
    residual stream also carries the earlier layers' difference `carried` (elementwise) into
    this output unchanged. Each element within carried + the bar's max-abs; relative L2 <= 1e-2."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    _, rl = metrics(gpu, ref)
    worst = float(np.max(err - np.asarray(carried)))
    log(f"  {what}: max(|err| - carried) {worst:.3e} rel-L2 {rl:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert worst <= MAX_ABS and rl <= REL_L2, f"{what}: max(|err| - carried) {worst:.3e} rel-L2 {rl:.3e}"


@functools.lru_cache(maxsize=1)
def weights():
    bits = synth.make_weights_bf16(seed=0)
    w64 = {k: synth.bf16_bits_to_f64(v) for k, v in bits.items()}
    return bits, w64


@functools.lru_cache(maxsize=2)
def layer(max_positions: int = 16384):
    bits, _ = weights()
    return binding.Layer(binding.weights_to_device(bits), max_positions=max_positions)


def assert_codes_valid(codes: np.ndarray, scales: np.ndarray, pre: np.ndarray, what: str,
                       delta: float = 1e-4, max_frac: float = 1e-2):
    """Quantised activations (E4M3FN codes + one float32 scale per 128 features) against the
    oracle's quantiser applied to the oracle's float64 pre-quantisation values.

    A code is decided by rounding t = pre / scale. The kernel computes pre in float32 from a
    K-long accumulation, so its t carries an absolute error of order 1e-5 of the group's
    largest |t| (448); where t sits that close to a rounding boundary the two sides may land
    on different codes. Checked: the scales agree to `delta` (relative), at most `max_frac` of
    the codes differ, and every code lies between the oracle's roundings of t - d and t + d with
    d = delta * 448 (rounding is monotone, so these bound every value the kernel could have
    rounded).
    """
    from oracle import fp8 as ofp8

    rc, rs = ofp8.quantize_1x128(pre)
    rel = np.abs(scales.astype(np.float64) / rs - 1.0)
    diff = codes != rc
    frac = float(diff.mean())
    log(f"  {what}: scale rel-diff max {rel.max():.2e}; {int(diff.sum())} of {diff.size} codes differ ({frac:.2e})")
    assert rel.max() <= delta, f"{what}: scales differ (rel {rel.max():.2e})"
    assert frac <= max_frac, f"{what}: {frac:.2e} of the codes differ"
    if diff.any():
        n = pre.shape[0]
        t = (pre.reshape(n, -1, 128) / rs[:, :, None]).reshape(pre.shape)[diff]
        d = delta * 448.0
        lo = ofp8.e4m3_value(ofp8.e4m3_encode(t - d))
        hi = ofp8.e4m3_value(ofp8.e4m3_encode(t + d))
        vg = ofp8.e4m3_value(codes[diff])
        bad = (vg < lo) | (vg > hi)
        if bad.any():
            k = np.flatnonzero(bad)[:8]
            log(f"  {what}: outliers t={t[k]} gpu={vg[k]} oracle={ofp8.e4m3_value(rc[diff][k])}")
        assert not bad.any(), f"{what}: {int(bad.sum())} codes lie outside the rounding of t +- {d:.3g}"


def y_of(t) -> np.ndarray:
    return synth.bf16_bits_to_f64(binding.tensor_to_bf16_bits(t))


def entries_f64(entry_bytes_rows) -> tuple[np.ndarray, np.ndarray]:
    """bf16 cache slots ([n, 1152] uint8, cpu numpy) -> (c_hat [n,512], k_pe [n,64]) float64."""
    bits = np.ascontiguousarray(entry_bytes_rows).view(np.uint16).reshape(-1, 576)
    v = synth.bf16_bits_to_f64(bits)
    return v[:, :512], v[:, 512:]


def oracle_cfg() -> omla.Config:
    return omla.KIMI_K2
