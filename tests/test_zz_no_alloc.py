"""mla_decode_static (the decode step on the library's static device scratch, for callers that
cannot allocate) against mla_decode on identical caches, through the C ABI.

Two calls in a row on the same caches, the second with fewer sequences and a shorter step
(so the scratch still holds the first call's larger values): outputs bit-identical to
mla_decode's and within the parity bar of the float64 oracle, cache bytes and lengths identical.
Also the FP8 layer (at 128 sequences of 16384 positions too), and a step too large for the scratch,
which is rejected before anything runs.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_close, layer, log, weights, y_of

pytestmark = pytest.mark.gpu


def _twin_caches(L, lens, seed):
    caches = [binding.Cache(L, [n + 2 for n in lens], fill_byte=0x77) for _ in range(2)]  # same bytes in unused slots
    ents = {}
    for s, n in enumerate(lens):
        if n:
            ents[s] = synth.make_cache_entries(n, seed=seed + s)
            for c in caches:
                L.cache_append(c, s, binding.bf16_tensor(ents[s]))
    return caches, ents


def test_static_decode_matches_decode_twice_bf16():
    import torch

    lens = [0, 65, 700, 2049, 300]
    log(f"static-scratch decode vs mla_decode, bf16, lens={lens}, then a smaller second call")
    _, w64 = weights()
    L = layer()
    (ca, cb), ents = _twin_caches(L, lens, seed=8000)
    calls = [np.array([3, 0, 4, 1, 2], dtype=np.int32), np.array([2, 1], dtype=np.int32)]
    xs = [synth.make_hidden(len(calls[0]), seed=8100), synth.make_hidden(len(calls[1]), seed=8101)]
    held = {s: (synth.bf16_bits_to_f64(ents[s]) if s in ents else np.zeros((0, 576))) for s in range(len(lens))}
    for k, (order, xbits) in enumerate(zip(calls, xs)):
        x = binding.bf16_tensor(xbits)
        ya = L.decode(ca, order, x)
        yb = L.decode_static(cb, order, x)
        torch.cuda.synchronize()
        assert np.array_equal(binding.tensor_to_bf16_bits(ya), binding.tensor_to_bf16_bits(yb)), f"call {k}: outputs differ"
        assert torch.equal(ca.data, cb.data), f"call {k}: cache bytes differ"
        assert ca.len_h.tolist() == cb.len_h.tolist() and torch.equal(ca.len_d, cb.len_d)
        yg = y_of(yb)
        for b, s in enumerate(order):
            e = held[s]
            ref = omla.forward(synth.bf16_bits_to_f64(xbits[b:b + 1]), w64, cache=(e[:, :512], e[:, 512:]))
            assert_close(yg[b:b + 1], ref["y"], f"call {k} seq {s} (L={e.shape[0]})")
            # the step's own entry (the oracle's) joins the sequence's cache for the next call
            held[s] = np.concatenate([e, np.concatenate([ref["c_hat"], ref["k_pe"]], axis=1)])


def test_static_decode_matches_decode_fp8():
    import torch

    from test_gpu_fp8 import fp8_setup, pack_fp8_entries

    lens = [100, 1500, 0]
    log(f"static-scratch decode vs mla_decode, FP8, lens={lens}, then a smaller second call")
    _, _, L = fp8_setup()
    ca, cb = (binding.Cache(L, [n + 2 for n in lens], fill_byte=0x77) for _ in range(2))
    for s, n in enumerate(lens):
        if n:
            e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=8200 + s))
            raw, _ = pack_fp8_entries(e[:, :512], e[:, 512:])
            for c in (ca, cb):
                L.cache_append(c, s, torch.from_numpy(raw).cuda())
    for k, order in enumerate([np.array([1, 2, 0], dtype=np.int32), np.array([0], dtype=np.int32)]):
        x = binding.bf16_tensor(synth.make_hidden(len(order), seed=8300 + k))
        ya = L.decode(ca, order, x)
        yb = L.decode_static(cb, order, x)
        torch.cuda.synchronize()
        assert np.array_equal(binding.tensor_to_bf16_bits(ya), binding.tensor_to_bf16_bits(yb)), f"call {k}: outputs differ"
        assert torch.equal(ca.data, cb.data) and ca.len_h.tolist() == cb.len_h.tolist()


def test_static_decode_fp8_128_sequences_of_16384():
    """The FP8 decode step at its full size (128 sequences of 16384 cached positions, 124.7 MiB of
    workspace) fits the scratch; then 64 of those sequences in another order."""
    import torch

    from test_gpu_fp8 import fp8_setup

    B, P = 128, 16384
    log(f"static-scratch decode vs mla_decode, FP8, {B} x {P}, then 64 sequences")
    wq, _, _ = fp8_setup()
    L = binding.Layer(binding.weights_to_device(wq), max_positions=P + 8, wdtype=binding.WDTYPE_FP8)
    base = torch.from_numpy(synth.make_cache_entries_fp8(P, seed=8500)).cuda()
    ca, cb = (binding.Cache(L, [P + 3] * B, fill_byte=0x55) for _ in range(2))
    for s in range(B):
        ents = torch.roll(base, shifts=97 * s, dims=0).contiguous()  # a different cache per sequence
        for c in (ca, cb):
            L.cache_append(c, s, ents)
    del base
    for k, order in enumerate([np.arange(B, dtype=np.int32), np.arange(B - 1, -1, -2, dtype=np.int32)]):
        x = binding.bf16_tensor(synth.make_hidden(len(order), seed=8600 + k))
        ya = L.decode(ca, order, x)
        yb = L.decode_static(cb, order, x)
        torch.cuda.synchronize()
        assert np.array_equal(binding.tensor_to_bf16_bits(ya), binding.tensor_to_bf16_bits(yb)), f"call {k}: outputs differ"
        assert torch.equal(ca.data, cb.data) and ca.len_h.tolist() == cb.len_h.tolist(), f"call {k}: caches differ"
        assert bool(torch.isfinite(yb.float()).all())


def test_static_decode_rejects_a_step_larger_than_its_scratch():
    import torch

    B = 1000
    log(f"static-scratch decode: {B} sequences need more than the 128 MiB scratch")
    L = layer()
    need = L.decode_workspace_bytes(B, B)
    assert need > 128 << 20
    cache = binding.Cache(L, [1] * B, fill_byte=0x3C)
    x = binding.bf16_tensor(synth.make_hidden(B, seed=8400))
    with pytest.raises(binding.MlaError) as ei:
        L.decode_static(cache, np.arange(B), x)
    assert ei.value.status == 5  # MLA_E_WORKSPACE
    torch.cuda.synchronize()
    assert np.all(cache.len_h == 0) and int(cache.len_d.sum()) == 0
    assert bool((cache.data == 0x3C).all())
