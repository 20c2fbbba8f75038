"""GPU parity with YaRN RoPE (the rope_scaling of the config excerpt on the "KV cache" page:
factor 32 over an original 4,096 positions, beta_fast = beta_slow = 1, mscale = mscale_all_dim = 1)
against the float64 oracle configured the same way. Only the rotary table and the softmax scale
change, so the cases cover the two places a position enters (the new entry's shared key and
the query's rotary part) on prefill and decode, below and beyond the original 4,096 positions.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_bf16_rounding_of, assert_close, entries_f64, log, weights, y_of

pytestmark = pytest.mark.gpu
YARN = omla.KIMI_K2_YARN


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def yarn_layer(torch_cuda):
    bits, _ = weights()
    return binding.Layer(binding.weights_to_device(bits), max_positions=8192, rope_scaling=binding.KIMI_K2_YARN)


def test_yarn_prefill_then_decode(torch_cuda, yarn_layer):
    log("YaRN: prefill 40 + 2 decode steps")
    L = yarn_layer
    _, w64 = weights()
    xbits = synth.make_hidden(42, seed=2101)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [48])
    y0 = L.prefill(cache, [0], [0, 40], xt[:40])
    ys = [y_of(L.decode(cache, [0], xt[40 + i:41 + i].contiguous())) for i in range(2)]
    torch_cuda.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    ref = omla.forward(x64, w64, cfg=YARN)
    assert_close(y_of(y0), ref["y"][:40], "YaRN prefill y")
    assert_close(np.concatenate(ys), ref["y"][40:], "YaRN decode y")
    # the cached shared keys are rotated with the YaRN table (and differ from plain RoPE's)
    c_gpu, k_gpu = entries_f64(cache.slots(0).cpu().numpy()[:42])
    c_ref, k_ref = omla.kv_entries(x64, w64, cfg=YARN)
    # bf16 slots: each value within one bf16 unit of the oracle's
    assert_bf16_rounding_of(k_gpu, k_ref, "YaRN cached k_pe")
    assert_bf16_rounding_of(c_gpu, c_ref, "YaRN cached c_hat")
    # the slowed pairs (20..31, features 40..63) have turned visibly less than under plain RoPE
    _, k_plain = omla.kv_entries(x64, w64)
    assert np.max(np.abs(k_ref[20:, 40:] - k_plain[20:, 40:])) > 0.05


def test_yarn_decode_beyond_original_context(torch_cuda, yarn_layer):
    """Decode of two sequences at positions 5000 and 6100 over cached synthetic entries."""
    log("YaRN: decode B=2 at positions 5000 and 6100")
    L = yarn_layer
    _, w64 = weights()
    lens = [5000, 6100]
    cache = binding.Cache(L, [n + 1 for n in lens])
    ents = []
    for s, n in enumerate(lens):
        e = synth.make_cache_entries(n, seed=2200 + s)
        L.cache_append(cache, s, binding.bf16_tensor(e))
        ents.append(synth.bf16_bits_to_f64(e))
    xn = synth.make_hidden(2, seed=2102)
    y = y_of(L.decode(cache, [0, 1], binding.bf16_tensor(xn)))
    torch_cuda.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xn)
    for s in range(2):
        ref = omla.forward(x64[s:s + 1], w64, cfg=YARN, cache=(ents[s][:, :512], ents[s][:, 512:]), absorbed=True)
        assert_close(y[s:s + 1], ref["y"], f"YaRN decode seq {s}")
    assert list(cache.len_h[:2]) == [5001, 6101]
