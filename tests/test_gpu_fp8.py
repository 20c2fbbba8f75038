"""GPU parity of the FP8 layer (E4M3FN weights with 128x128 block scales, dynamic 1x128
activation quantisation) against the float64 oracle in W8A8 mode.

The oracle dequantises the weights exactly and passes every projection input through the same
quantiser definition (per token, per 128-feature group, s = fl32(amax/448), RNE-saturated
e4m3 codes); both sides quantise from float32 values, so codes agree except where the GPU's and
the oracle's float32 inputs fall on opposite sides of a rounding boundary.
Bar: max-abs-err <= 2e-2 and relative L2 <= 1e-2 on the bf16 outputs.
"""
import functools

import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import fp8 as ofp8
from oracle import mla as omla

from gpu_common import assert_close, assert_codes_valid, log, y_of

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def fp8_setup():
    wq = synth.make_weights_fp8(seed=0)
    w64 = {}
    for name in ("q_a", "q_b", "kv_a", "kv_b", "o"):
        w64[name] = ofp8.dequant_weight(wq[name], wq[name + "_s"])
    for name in ("q_a_norm", "kv_a_norm"):
        w64[name] = synth.bf16_bits_to_f64(wq[name])
    layer = binding.Layer(binding.weights_to_device(wq), max_positions=8192, wdtype=binding.WDTYPE_FP8)
    return wq, w64, layer


def pack_fp8_entries(c_hat: np.ndarray, k_pe: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Oracle-quantised latent + float32 rotary key -> 784-byte cache slots, and the latent the
    oracle attends over (the dequantised codes)."""
    codes, scales = ofp8.quantize_1x128(c_hat)
    n = c_hat.shape[0]
    out = np.zeros((n, 784), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:528] = scales.astype(np.float32).view(np.uint8).reshape(n, 16)
    out[:, 528:] = np.ascontiguousarray(k_pe.astype(np.float32)).view(np.uint8).reshape(n, 256)
    return out, ofp8.dequant_1x128(codes, scales)


def unpack_fp8_entries(raw: np.ndarray):
    codes = raw[:, :512]
    scales = np.ascontiguousarray(raw[:, 512:528]).view(np.float32).reshape(-1, 4)
    kpe = np.ascontiguousarray(raw[:, 528:]).view(np.float32).reshape(-1, 64).astype(np.float64)
    return ofp8.dequant_1x128(codes, scales), kpe


@pytest.mark.parametrize("lens_t", [[64], [100], [300], [50, 129]])
def test_fp8_prefill_matches_w8a8_oracle(lens_t):
    import torch

    log(f"fp8 prefill lens={lens_t}")
    wq, w64, L = fp8_setup()
    q_start = np.concatenate([[0], np.cumsum(lens_t)]).astype(np.int32)
    xbits = synth.make_hidden(int(q_start[-1]), seed=4000 + sum(lens_t))
    cache = binding.Cache(L, lens_t)
    y = y_of(L.prefill(cache, np.arange(len(lens_t)), q_start, binding.bf16_tensor(xbits)))
    torch.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    for b, t in enumerate(lens_t):
        rows = slice(q_start[b], q_start[b + 1])
        ref = omla.forward(x64[rows], w64, w8a8=True)
        assert_close(y[rows], ref["y"], f"seq {b} (T={t}) y")
        raw = cache.slots(b).cpu().numpy()
        _, k_gpu = unpack_fp8_entries(raw)
        c_pre = omla.rmsnorm(ref["ckv"][:, :512], w64["kv_a_norm"], omla.KIMI_K2.eps)
        assert_codes_valid(raw[:, :512], np.ascontiguousarray(raw[:, 512:528]).view(np.float32).reshape(-1, 4),
                           c_pre, f"seq {b} cached c_hat codes")
        assert_close(k_gpu, ref["k_pe"], f"seq {b} cached k_pe (float32)", max_abs=5e-4, rel_l2=1e-4)


def test_fp8_decode_matches_w8a8_oracle():
    import torch

    lens = [0, 1, 100, 1500]
    log(f"fp8 decode lens={lens}")
    wq, w64, L = fp8_setup()
    cache = binding.Cache(L, [n + 1 for n in lens])
    lat = {}
    for s, n in enumerate(lens):
        if n:
            e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=5000 + s))
            raw, c_dq = pack_fp8_entries(e[:, :512], e[:, 512:])
            lat[s] = (c_dq, e[:, 512:].astype(np.float32).astype(np.float64))
            L.cache_append(cache, s, torch.from_numpy(raw).cuda())
    xn = synth.make_hidden(len(lens), seed=5100)
    y = y_of(L.decode(cache, np.arange(len(lens)), binding.bf16_tensor(xn)))
    torch.cuda.synchronize()
    for s, n in enumerate(lens):
        kw = {"cache": lat[s]} if n else {}
        ref = omla.forward(synth.bf16_bits_to_f64(xn[s:s + 1]), w64, w8a8=True, **kw)
        assert_close(y[s:s + 1], ref["y"], f"seq {s} (L={n})")


@pytest.mark.parametrize("B", [100, 130])
def test_fp8_decode_many_sequences(B):
    """100 sequences: the q_a|kv_a partial sums of the K-split projection go to the norm kernel as
    parts (up to 128 rows). 130: more sequences than the per-head absorb kernel pairs (it adds the
    query's two absorbed products itself for up to 128), so the attention kernel adds them, and the
    projection's partial sums go through its own reduction."""
    import torch

    lens = [(7 * s) % 41 for s in range(B)]
    log(f"fp8 decode B={B}, lengths 0..40")
    wq, w64, L = fp8_setup()
    cache = binding.Cache(L, [n + 1 for n in lens])
    lat = {}
    for s, n in enumerate(lens):
        if n:
            e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=5300 + s))
            raw, c_dq = pack_fp8_entries(e[:, :512], e[:, 512:])
            lat[s] = (c_dq, e[:, 512:].astype(np.float32).astype(np.float64))
            L.cache_append(cache, s, torch.from_numpy(raw).cuda())
    xn = synth.make_hidden(B, seed=5310)
    y = y_of(L.decode(cache, np.arange(B), binding.bf16_tensor(xn)))
    torch.cuda.synchronize()
    for s in (0, 1, 64, B - 3, B - 2, B - 1):
        kw = {"cache": lat[s]} if lens[s] else {}
        ref = omla.forward(synth.bf16_bits_to_f64(xn[s:s + 1]), w64, w8a8=True, **kw)
        assert_close(y[s:s + 1], ref["y"], f"seq {s} (L={lens[s]})")


def test_fp8_prefill_then_decode():
    import torch

    log("fp8 prefill 40 + 2 decode steps")
    wq, w64, L = fp8_setup()
    xbits = synth.make_hidden(42, seed=5200)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [48])
    L.prefill(cache, [0], [0, 40], xt[:40])
    ys = [y_of(L.decode(cache, [0], xt[40 + i:41 + i].contiguous())) for i in range(2)]
    torch.cuda.synchronize()
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w64, rows=np.arange(40, 42), w8a8=True)
    assert_close(np.concatenate(ys), ref["y"], "fp8 decode steps after prefill")
