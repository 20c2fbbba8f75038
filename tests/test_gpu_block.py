"""GPU parity of the attention half of a decoder block (mla_block_prefill / mla_block_decode):
h = x + MLA(xn), xn the block's input RMSNorm in bf16 ("Attention input" page, block and
rmsnorm excerpts), against the float64 oracle's block_attention on the same seeded inputs.

Bar: max-abs-err <= 2e-2 and relative L2 <= 1e-2 on h (bf16) against the oracle's unrounded
x + y, and on h - x (the attention's contribution, which the residual would otherwise dominate)
against y.
"""
import functools

import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import fp8 as ofp8
from oracle import mla as omla

from gpu_common import assert_close, layer, log, weights, y_of

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def norm_gain():
    bits = synth.make_block_norm(seed=7)
    return bits, synth.bf16_bits_to_f64(bits)


def check_block(h_gpu, x64, ref, what):
    # the oracle's h is its bf16 rounding of x + y; the GPU's h is its own rounding of x + y_gpu, so
    # each is held against the unrounded sum (the GPU's rounding counts as its error)
    assert_close(h_gpu, x64 + ref["y"], f"{what} h")
    assert_close(h_gpu - x64, ref["y"], f"{what} h - x", max_abs=2e-2, rel_l2=1e-2)


@pytest.mark.parametrize("in_place", [False, True])
def test_block_prefill_then_decode_bf16(in_place):
    import torch

    log(f"block bf16: prefill 40 + 2 decode steps, in_place={in_place}")
    _, w64 = weights()
    gbits, g64 = norm_gain()
    L = layer()
    g = binding.bf16_tensor(gbits)
    xbits = synth.make_hidden(42, seed=6000)
    x = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [48])
    xp = x[:40].clone()
    hp = L.block_prefill(cache, [0], [0, 40], g, xp, h=xp if in_place else None)
    hs = [hp]
    for i in range(2):
        xd = x[40 + i:41 + i].clone()
        hs.append(L.block_decode(cache, [0], g, xd, h=xd if in_place else None))
    torch.cuda.synchronize()
    h = np.concatenate([y_of(t) for t in hs])
    x64 = synth.bf16_bits_to_f64(xbits)
    ref = omla.block_attention(x64, w64, g64)
    check_block(h, x64, ref, "prefill+decode")
    assert int(cache.len_h[0]) == 42


def test_block_ragged_prefill_and_batched_decode_bf16():
    import torch

    lens_t = [17, 64, 5]
    log(f"block bf16: ragged prefill {lens_t} + one batched decode step")
    _, w64 = weights()
    gbits, g64 = norm_gain()
    L = layer()
    g = binding.bf16_tensor(gbits)
    q_start = np.concatenate([[0], np.cumsum(lens_t)]).astype(np.int32)
    xbits = synth.make_hidden(int(q_start[-1]) + len(lens_t), seed=6100)
    x = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [t + 1 for t in lens_t])
    n = int(q_start[-1])
    hp = y_of(L.block_prefill(cache, np.arange(3), q_start, g, x[:n]))
    hd = y_of(L.block_decode(cache, np.arange(3), g, x[n:].contiguous()))
    torch.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    for b, t in enumerate(lens_t):
        rows = np.concatenate([np.arange(q_start[b], q_start[b + 1]), [n + b]])
        ref = omla.block_attention(x64[rows], w64, g64)
        got = np.concatenate([hp[q_start[b]:q_start[b + 1]], hd[b:b + 1]])
        check_block(got, x64[rows], ref, f"seq {b} (T={t})")


def test_block_fp8_prefill_then_decode():
    import torch

    log("block fp8: prefill 33 + 1 decode step")
    wq = synth.make_weights_fp8(seed=0)
    w64 = {}
    for name in ("q_a", "q_b", "kv_a", "kv_b", "o"):
        w64[name] = ofp8.dequant_weight(wq[name], wq[name + "_s"])
    for name in ("q_a_norm", "kv_a_norm"):
        w64[name] = synth.bf16_bits_to_f64(wq[name])
    L = binding.Layer(binding.weights_to_device(wq), max_positions=4096, wdtype=binding.WDTYPE_FP8)
    gbits, g64 = norm_gain()
    g = binding.bf16_tensor(gbits)
    xbits = synth.make_hidden(34, seed=6200)
    x = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [40])
    hp = y_of(L.block_prefill(cache, [0], [0, 33], g, x[:33]))
    hd = y_of(L.block_decode(cache, [0], g, x[33:].contiguous()))
    torch.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    ref = omla.block_attention(x64, w64, g64, w8a8=True)
    check_block(np.concatenate([hp, hd]), x64, ref, "fp8 prefill+decode")
    L.close()


def test_block_fp8_prefill_1100_tokens_sampled_rows():
    """A prefill long enough for the prefill-sized FP8 o_proj, whose epilogue adds the residual
    before the bf16 rounding (in place: h overwrites x)."""
    import torch

    T = 1100
    log(f"block fp8: prefill {T} tokens in place, sampled rows")
    wq = synth.make_weights_fp8(seed=0)
    w64 = {}
    for name in ("q_a", "q_b", "kv_a", "kv_b", "o"):
        w64[name] = ofp8.dequant_weight(wq[name], wq[name + "_s"])
    for name in ("q_a_norm", "kv_a_norm"):
        w64[name] = synth.bf16_bits_to_f64(wq[name])
    L = binding.Layer(binding.weights_to_device(wq), max_positions=4096, wdtype=binding.WDTYPE_FP8)
    gbits, g64 = norm_gain()
    g = binding.bf16_tensor(gbits)
    xbits = synth.make_hidden(T, seed=6250)
    x = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [T])
    h = y_of(L.block_prefill(cache, [0], [0, T], g, x, h=x))
    torch.cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(xbits)
    rows = np.array([0, 1, 517, 1023, 1024, 1099])
    ref = omla.block_attention(x64, w64, g64, rows=rows, w8a8=True)
    check_block(h[rows], x64[rows], ref, f"fp8 prefill T={T} rows {rows.tolist()}")
    L.close()


def test_block_rejects_partial_overlap_and_missing_gain():
    import ctypes

    import torch

    log("block argument errors")
    L = layer()
    gbits, _ = norm_gain()
    g = binding.bf16_tensor(gbits)
    buf = binding.bf16_tensor(synth.make_hidden(8, seed=6300))
    cache = binding.Cache(L, [8])
    with pytest.raises(binding.MlaError, match="overlap"):
        L.block_prefill(cache, [0], [0, 4], g, buf[:4], h=buf[1:5])
    assert int(cache.len_h[0]) == 0
    lib = binding.lib()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    sid = np.zeros(1, dtype=np.int32)
    sid_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = lib.mla_block_decode(L.ctx, ctypes.byref(cache.desc), sid.ctypes.data, ctypes.c_void_p(sid_d.data_ptr()), 1,
                              None, ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(buf.data_ptr()),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == 1 and int(cache.len_h[0]) == 0
