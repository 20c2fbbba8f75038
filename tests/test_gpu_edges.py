"""GPU parity on the edge cases of the attention kernels, against the float64 oracle.

  * a peaked softmax: planted cache entries whose latent points along one head's absorbed query
    (c_hat_p = beta q_lat / |q_lat|, k_pe_p = 0), so that head's score at position p lies about
    20 log2 units above every other score it sees. When the key block holding p arrives, the
    block maximum exceeds the running maximum by far more than the kernels' lazy-rescale margin
    (8 log2 units): the output accumulators, which already hold the earlier blocks, are rescaled;
    a decode's split holding p ends with a maximum far above its sibling splits', so the merge
    combines very different maxima. Checked on the inputs themselves (from the oracle's scores)
    that the jump occurs. Chunked bf16 prefill onto a planted prefix, bf16 varlen decode, FP8
    decode. (The scores keep the layer's softmax scale: raising the scale itself to 1.0 spreads
    every score over tens of log2 units, and then bf16 operands alone -- the rounding of q, K and
    V, emulated on the CPU -- move the output by max-abs 4.9e-2 / rel-L2 1.1e-2, past the bar,
    whatever the kernel does.)
  * uniform attention (q_b = 0: every score is 0, so each query averages the values of all the
    positions it sees), prefill followed by a decode step;
  * chunked prefill of 300 tokens (three query tiles) onto 1,500 cached positions (not a multiple
    of the 64-key block).

Bar: max-abs-err <= 2e-2 and relative L2 <= 1e-2 on the bf16 outputs.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_close, layer, log, weights, y_of
from test_gpu_fp8 import fp8_setup, pack_fp8_entries

pytestmark = pytest.mark.gpu

LAZY_MARGIN = 8.0   # log2 units
PLANT_LOG2 = 20.0   # planted score, log2 units (typical scores here stay within about 5)
SIGMA = omla.KIMI_K2.sigma


def q_lat_of(q_nope_row, w_kvb):
    """Absorbed queries W_UK,h^T q_nope,h of one token, [heads, 512]."""
    wk = w_kvb.reshape(64, 256, 512)
    return np.einsum("hd,hdc->hc", q_nope_row, wk[:, :128, :])


def plant(ent, plants):
    """Planted entries (float64 [n, 576]): for each (position, q_lat vector of the target head),
    c_hat_p along q_lat with the length that puts the head's score at PLANT_LOG2, k_pe_p = 0."""
    ent = ent.copy()
    for p, q in plants:
        beta = PLANT_LOG2 * np.log(2.0) / (SIGMA * np.linalg.norm(q))
        ent[p, :512] = beta * q / np.linalg.norm(q)
        ent[p, 512:] = 0.0
    return ent


def scores_log2(q_nope_row, q_pe_row, c_hat, k_pe, w_kvb):
    """Oracle scores of one query row in log2 units, [heads, positions]."""
    return (q_lat_of(q_nope_row, w_kvb) @ c_hat.T + q_pe_row @ k_pe.T) * SIGMA / np.log(2.0)


def largest_jump(s, block):
    """Largest amount by which a key block's maximum exceeds the running maximum of the blocks
    before it (over heads), scanning from key 0 as the kernels do."""
    nb = -(-s.shape[1] // block)
    bmax = np.stack([s[:, b * block:(b + 1) * block].max(axis=1) for b in range(nb)], axis=1)
    run = np.maximum.accumulate(bmax, axis=1)
    return float(np.max(bmax[:, 1:] - run[:, :-1])) if nb > 1 else 0.0


def test_peaked_softmax_chunked_prefill_bf16():
    import torch

    l0, T = 700, 300
    log(f"peaked softmax: bf16 prefill of {T} tokens onto {l0} planted cached positions")
    _, w64 = weights()
    L = layer()
    xbits = synth.make_hidden(T, seed=7000)
    x64 = synth.bf16_bits_to_f64(xbits)
    qp = omla.query_path(x64, w64, l0 + np.arange(T))  # q_nope does not depend on the position
    targets = [(299, 5, 400), (150, 33, 520), (10, 60, 690)]  # (token, head, planted position)
    prefix = synth.bf16_bits_to_f64(synth.make_cache_entries(l0, seed=7001))
    prefix = plant(prefix, [(p, q_lat_of(qp["q_nope"][t], w64["kv_b"])[h]) for t, h, p in targets])
    pbits = synth.f32_to_bf16_bits(prefix.astype(np.float32))
    prefix = synth.bf16_bits_to_f64(pbits)
    cache = binding.Cache(L, [l0 + T])
    L.cache_append(cache, 0, binding.bf16_tensor(pbits))
    y = y_of(L.prefill(cache, [0], [0, T], binding.bf16_tensor(xbits)))
    torch.cuda.synchronize()
    ref = omla.forward(x64, w64, cache=(prefix[:, :512], prefix[:, 512:]), absorbed=True)
    c = np.concatenate([prefix[:, :512], ref["c_hat"]])
    k = np.concatenate([prefix[:, 512:], ref["k_pe"]])
    for t, h, p in targets:
        s = scores_log2(ref["q_nope"][t], ref["q_pe"][t], c[:l0 + t + 1], k[:l0 + t + 1], w64["kv_b"])
        jump = largest_jump(s[h:h + 1], 64)
        log(f"  token {t} head {h}: planted key at {p}, block-maximum jump {jump:.1f} log2 units")
        assert jump > LAZY_MARGIN
    assert_close(y, ref["y"], "peaked prefill y")


def test_peaked_softmax_decode_varlen_bf16():
    import torch

    lens = [0, 1, 63, 64, 65, 700, 2049]
    targets = {5: [(7, 680)], 6: [(30, 1330), (61, 1700)]}  # sequence -> (head, planted position)
    log(f"peaked softmax: bf16 decode lens={lens}, planted keys {targets}")
    _, w64 = weights()
    L = layer()
    order = np.array([6, 0, 5, 2, 1, 4, 3], dtype=np.int32)
    xn = synth.make_hidden(len(order), seed=7200)
    x64 = synth.bf16_bits_to_f64(xn)
    cache = binding.Cache(L, [n + 1 for n in lens])
    ents = {}
    for b, s in enumerate(order):
        n = lens[s]
        if not n:
            continue
        e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=7100 + s))
        if s in targets:
            qn = omla.query_path(x64[b:b + 1], w64, np.array([n]))["q_nope"][0]
            e = plant(e, [(p, q_lat_of(qn, w64["kv_b"])[h]) for h, p in targets[s]])
        ebits = synth.f32_to_bf16_bits(e.astype(np.float32))
        ents[s] = synth.bf16_bits_to_f64(ebits)
        L.cache_append(cache, s, binding.bf16_tensor(ebits))
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn)))
    torch.cuda.synchronize()
    for b, s in enumerate(order):
        kw = dict(cache=(ents[s][:, :512], ents[s][:, 512:])) if lens[s] else {}
        ref = omla.forward(x64[b:b + 1], w64, **kw)
        for h, p in targets.get(s, []):
            c = np.concatenate([ents[s][:, :512], ref["c_hat"]])
            k = np.concatenate([ents[s][:, 512:], ref["k_pe"]])
            jump = largest_jump(scores_log2(ref["q_nope"][0], ref["q_pe"][0], c, k, w64["kv_b"])[h:h + 1], 32)
            log(f"  seq {s} head {h}: planted key at {p}, block-maximum jump {jump:.1f} log2 units")
            assert jump > LAZY_MARGIN
        assert_close(y[b:b + 1], ref["y"], f"seq {s} (L={lens[s]})")


def test_peaked_softmax_decode_fp8():
    import torch

    lens = [0, 100, 1500]
    targets = {1: [(12, 97)], 2: [(40, 1070), (3, 1300)]}
    log(f"peaked softmax: FP8 decode lens={lens}, planted keys {targets}")
    wq, w64, L = fp8_setup()
    xn = synth.make_hidden(len(lens), seed=7400)
    x64 = synth.bf16_bits_to_f64(xn)
    cache = binding.Cache(L, [n + 1 for n in lens])
    lat = {}
    for s, n in enumerate(lens):
        if not n:
            continue
        e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=7300 + s))
        if s in targets:
            qn = omla.query_path(x64[s:s + 1], w64, np.array([n]), w8a8=True)["q_nope"][0]
            e = plant(e, [(p, q_lat_of(qn, w64["kv_b"])[h]) for h, p in targets[s]])
        raw, c_dq = pack_fp8_entries(e[:, :512], e[:, 512:])
        lat[s] = (c_dq, e[:, 512:].astype(np.float32).astype(np.float64))
        L.cache_append(cache, s, torch.from_numpy(raw).cuda())
    y = y_of(L.decode(cache, np.arange(len(lens)), binding.bf16_tensor(xn)))
    torch.cuda.synchronize()
    for s, n in enumerate(lens):
        kw = {"cache": lat[s]} if n else {}
        ref = omla.forward(x64[s:s + 1], w64, w8a8=True, **kw)
        for h, p in targets.get(s, []):
            c = np.concatenate([lat[s][0], ref["c_hat"]])
            k = np.concatenate([lat[s][1], ref["k_pe"]])
            jump = largest_jump(scores_log2(ref["q_nope"][0], ref["q_pe"][0], c, k, w64["kv_b"])[h:h + 1], 32)
            log(f"  seq {s} head {h}: planted key at {p}, block-maximum jump {jump:.1f} log2 units")
            assert jump > LAZY_MARGIN
        assert_close(y[s:s + 1], ref["y"], f"seq {s} (L={n})")


def test_uniform_attention_when_q_b_vanishes():
    import torch

    log("uniform attention (q_b = 0): prefill 200 + one decode step")
    bits, w64 = weights()
    zbits = dict(bits)
    zbits["q_b"] = np.zeros_like(bits["q_b"])
    w0 = dict(w64)
    w0["q_b"] = np.zeros_like(w64["q_b"])
    L = binding.Layer(binding.weights_to_device(zbits), max_positions=4096)
    xbits = synth.make_hidden(201, seed=7500)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [201])
    yp = y_of(L.prefill(cache, [0], [0, 200], xt[:200]))
    yd = y_of(L.decode(cache, [0], xt[200:].contiguous()))
    torch.cuda.synchronize()
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w0)
    # the oracle's closed form (pinned on the CPU): the mean of the values of positions 0..t
    _, v = omla.rebuild_kv(ref["c_hat"], ref["k_pe"], w64["kv_b"])
    o_mean = (np.cumsum(v, axis=0) / np.arange(1, 202)[:, None, None]).reshape(201, -1)
    assert np.allclose(ref["y"], o_mean @ w64["o"].T, rtol=0, atol=1e-10)
    assert_close(yp, ref["y"][:200], "uniform prefill y")
    assert_close(yd, ref["y"][200:], "uniform decode y")
    L.close()


def test_chunked_prefill_300_onto_1500():
    import torch

    l0, t = 1500, 300
    log(f"chunked prefill {t} onto {l0} cached positions")
    _, w64 = weights()
    L = layer()
    xbits = synth.make_hidden(l0 + t, seed=7600)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [l0 + t])
    L.prefill(cache, [0], [0, l0], xt[:l0])
    y2 = y_of(L.prefill(cache, [0], [0, t], xt[l0:].contiguous()))
    torch.cuda.synchronize()
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w64, rows=np.arange(l0, l0 + t), absorbed=True)
    assert_close(y2, ref["y"], "second chunk y")
    assert cache.len_h[0] == l0 + t and int(cache.len_d[0]) == l0 + t
