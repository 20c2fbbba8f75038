"""GPU check of a two-layer stack over one cache pool (mla_cache_pool_plan / mla_cache_pool_layer):
decoder-block attention halves of two layers with their own weights, each layer's cache carved from
the same buffer with the shared slot layout, against the float64 oracle chaining block_attention
through both layers. The oracle's chain passes bf16 hidden states between the layers, as the model
does (each block returns a bf16 tensor); nothing from the GPU enters the reference.

Checked layer by layer at the single-layer bar (max-abs-err 2e-2, relative L2 1e-2):
  * layer 0: h0 against the oracle's unrounded x + y0 (the GPU's rounding counts as its error);
  * layer 1: its contribution h1 - h0 (GPU values on both sides of the difference) against the
    oracle's unrounded y1; h1 itself against the oracle's h0 + y1, within the same bar plus the
    elementwise difference the residual stream carries over from layer 0 (|h0_gpu - h0_oracle|);
  * the second layer's cached latent entries at their place in the pool, at the bar;
  * padding slots of both layers untouched.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_close, assert_close_carried, entries_f64, layer, log, weights, y_of

pytestmark = pytest.mark.gpu

FILL = 0xAB


def test_two_layer_stack_over_one_pool():
    import torch

    lens_t = [20, 9]
    log(f"two-layer pool: prefill {lens_t} then one decode step through both layers")
    _, w0 = weights()
    L0 = layer()
    bits1 = synth.make_weights_bf16(seed=1)
    w1 = {k: synth.bf16_bits_to_f64(v) for k, v in bits1.items()}
    L1 = binding.Layer(binding.weights_to_device(bits1), max_positions=16384)
    g_bits = [synth.make_block_norm(seed=7), synth.make_block_norm(seed=8)]
    g = [binding.bf16_tensor(b) for b in g_bits]
    g64 = [synth.bf16_bits_to_f64(b) for b in g_bits]

    caps = [t + 1 for t in lens_t]
    pool = binding.CachePool(L0.cfg, 2, caps, align=16, fill_byte=FILL)
    assert pool.layer_bytes == pool.total_slots * 1152 and pool.pool_bytes == 2 * pool.layer_bytes
    c0, c1 = pool.layer(0), pool.layer(1)

    q_start = np.concatenate([[0], np.cumsum(lens_t)]).astype(np.int32)
    n = int(q_start[-1])
    xbits = synth.make_hidden(n + len(lens_t), seed=6400)
    x = binding.bf16_tensor(xbits)
    sids = np.arange(len(lens_t))
    h0p = L0.block_prefill(c0, sids, q_start, g[0], x[:n])
    h1p = L1.block_prefill(c1, sids, q_start, g[1], h0p)
    h0d = L0.block_decode(c0, sids, g[0], x[n:].contiguous())
    h1d = L1.block_decode(c1, sids, g[1], h0d)
    torch.cuda.synchronize()
    h0 = np.concatenate([y_of(h0p), y_of(h0d)])
    h1 = np.concatenate([y_of(h1p), y_of(h1d)])
    raw = pool.pool.cpu().numpy()
    L1.close()

    x64 = synth.bf16_bits_to_f64(xbits)
    for b, t in enumerate(lens_t):
        rows = np.concatenate([np.arange(q_start[b], q_start[b + 1]), [n + b]])
        r0 = omla.block_attention(x64[rows], w0, g64[0])
        r1 = omla.block_attention(r0["h"], w1, g64[1])
        g0, g1 = h0[rows], h1[rows]
        assert_close(g0, x64[rows] + r0["y"], f"seq {b} (T={t}) layer 0 h")
        assert_close(g1 - g0, r1["y"], f"seq {b} layer 1 contribution h1 - h0")
        assert_close_carried(g1, r0["h"] + r1["y"], np.abs(g0 - r0["h"]), f"seq {b} layer 1 h")
        # the second layer's entries sit at layer_bytes + offset * 1152 in the pool
        o = int(pool.offset_h[b])
        ent = raw[pool.layer_bytes + o * 1152: pool.layer_bytes + (o + t + 1) * 1152].reshape(t + 1, 1152)
        c_gpu, k_gpu = entries_f64(ent)
        assert_close(c_gpu, r1["c_hat"], f"seq {b} layer-1 cached c_hat")
        assert_close(k_gpu, r1["k_pe"], f"seq {b} layer-1 cached k_pe")
    # padding slots after each sequence's positions are untouched in both layers
    for l in range(2):
        base = l * pool.layer_bytes
        for b, t in enumerate(lens_t):
            start = int(pool.offset_h[b]) + t + 1
            end = int(pool.offset_h[b + 1]) if b + 1 < len(lens_t) else pool.total_slots
            assert np.all(raw[base + start * 1152: base + end * 1152] == FILL), (l, b)
    assert c0.len_h.tolist() == caps and c1.len_h.tolist() == caps
