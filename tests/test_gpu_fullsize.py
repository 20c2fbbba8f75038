"""GPU parity at the full sizes of the layer's workloads, on sampled outputs.

The oracle computes the sampled rows one by one in the latent (absorbed) form of attention,
which its pins tie to the rebuilt form; the GPU runs the whole workload in one call, in the same
launch configuration the benchmark times.

  * prefill of 8192 tokens on an empty cache (bf16 weights);
  * batched decode of 64 sequences with cached lengths uniform in [1024, 8192] (bf16);
  * FP8 (E4M3 weights, 128x128 block scales, dynamic 1x128 activations): decode of 128
    sequences with 16384 cached positions each, and prefill of 4 sequences of 4096 tokens.

Long caches hold synthetic entries (the latent stands for RMSNorm outputs, the rotary key for a
projection of N(0,1) inputs); for FP8 the oracle's quantiser packs the entries, the sampled
sequences and their neighbours get caches of their own and the others share one, and every
sequence gets its own new token.
Bar: max-abs-err <= 2e-2 and relative L2 <= 1e-2 on the bf16 outputs.
"""
import functools

import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_bf16_rounding_of, assert_close, entries_f64, layer, log, weights, y_of
from test_gpu_fp8 import fp8_setup, pack_fp8_entries

pytestmark = pytest.mark.gpu


def test_prefill_8192_tokens_sampled_rows():
    import torch

    T = 8192
    log(f"full-size prefill T={T} (bf16)")
    bits, w64 = weights()
    L = layer()
    xbits = synth.make_hidden(T, seed=1003)
    cache = binding.Cache(L, [T])
    y = y_of(L.prefill(cache, [0], [0, T], binding.bf16_tensor(xbits)))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 2047, 4095, 6001, T - 1])
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w64, rows=rows, absorbed=True)
    assert_close(y[rows], ref["y"], f"y at rows {rows.tolist()}")
    c_gpu, k_gpu = entries_f64(cache.slots(0).cpu().numpy()[rows])
    assert_bf16_rounding_of(c_gpu, ref["c_hat"][rows], "cached c_hat at the sampled positions")
    assert_bf16_rounding_of(k_gpu, ref["k_pe"][rows], "cached k_pe at the sampled positions")


def test_decode_64_sequences_lengths_1024_to_8192():
    import torch

    B = 64
    lens = synth.make_lengths(B, 1024, 8192, seed=1002)
    log(f"full-size decode B={B}, cached lengths {int(lens.min())}..{int(lens.max())}, sum {int(lens.sum())}")
    bits, w64 = weights()
    L = layer()
    cache = binding.Cache(L, lens + 1)
    ents = {}
    for s in range(B):
        e = synth.make_cache_entries(int(lens[s]), seed=6000 + s)
        ents[s] = e
        L.cache_append(cache, s, binding.bf16_tensor(e))
    xn = synth.make_hidden(B, seed=1004)
    order = np.random.default_rng(7).permutation(B).astype(np.int32)  # batch order != sequence ids
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn[order])))
    torch.cuda.synchronize()
    sampled = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 5, 21, 40, 63})
    pos_of = {int(s): i for i, s in enumerate(order)}
    for s in sampled:
        e = synth.bf16_bits_to_f64(ents[s])
        ref = omla.forward(synth.bf16_bits_to_f64(xn[s:s + 1]), w64, cache=(e[:, :512], e[:, 512:]), absorbed=True)
        assert_close(y[pos_of[s]:pos_of[s] + 1], ref["y"], f"seq {s} (L={int(lens[s])})")
    assert np.all(cache.len_d.cpu().numpy() == lens + 1)


@functools.lru_cache(maxsize=1)
def fp8_long_layer():
    wq, w64, _ = fp8_setup()
    return binding.Layer(binding.weights_to_device(wq), max_positions=16448, wdtype=binding.WDTYPE_FP8)


def test_fp8_decode_128_sequences_16384_positions():
    import torch

    B, P = 128, 16384
    own = (0, 1, 76, 77, 78, 126, 127)  # the sampled sequences and their neighbours
    log(f"full-size FP8 decode B={B}, {P} cached positions each; distinct caches for {own}")
    wq, w64, _ = fp8_setup()
    L = fp8_long_layer()
    cache = binding.Cache(L, [P + 1] * B)

    def entries(seed):
        e = synth.bf16_bits_to_f64(synth.make_cache_entries(P, seed=seed))
        raw, c_dq = pack_fp8_entries(e[:, :512], e[:, 512:])
        return torch.from_numpy(raw).cuda(), (c_dq, e[:, 512:].astype(np.float32).astype(np.float64))

    base_t, base_ref = entries(5300)
    refs = {}
    for s in range(B):
        if s in own:
            t, refs[s] = entries(5301 + s)
            L.cache_append(cache, s, t)
        else:
            L.cache_append(cache, s, base_t)
    refs[40] = base_ref
    xn = synth.make_hidden(B, seed=5400)
    order = np.random.default_rng(9).permutation(B).astype(np.int32)  # batch order != sequence ids
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn[order])))
    torch.cuda.synchronize()
    pos_of = {int(s): i for i, s in enumerate(order)}
    for s in (0, 77, B - 1, 40):
        ref = omla.forward(synth.bf16_bits_to_f64(xn[s:s + 1]), w64, cache=refs[s], w8a8=True, absorbed=True)
        assert_close(y[pos_of[s]:pos_of[s] + 1], ref["y"], f"seq {s} (L={P})")
    assert np.all(cache.len_d.cpu().numpy() == P + 1)


def test_fp8_prefill_4_sequences_4096_tokens():
    import torch

    B, T = 4, 4096
    log(f"full-size FP8 prefill B={B} x T={T}")
    wq, w64, _ = fp8_setup()
    L = fp8_long_layer()
    xbits = synth.make_hidden(B * T, seed=5500)
    q_start = np.arange(B + 1, dtype=np.int32) * T
    cache = binding.Cache(L, [T] * B)
    y = y_of(L.prefill(cache, np.arange(B), q_start, binding.bf16_tensor(xbits)))
    torch.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    rows = np.array([0, 1000, T - 1])
    for b in (0, B - 1):
        ref = omla.forward(x64[b * T:(b + 1) * T], w64, rows=rows, w8a8=True, absorbed=True)
        assert_close(y[b * T + rows], ref["y"], f"seq {b} rows {rows.tolist()}")
