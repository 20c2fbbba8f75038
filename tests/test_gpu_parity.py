"""GPU parity of the MLA layer (HIP path through the C ABI) against the float64 CPU oracle.

Sizes here finish in seconds on the oracle and still span several query tiles, key blocks and
ragged tails. Parity bar on bf16 outputs: max-abs-err <= 2e-2 and relative L2 <= 1e-2;
cache slot contents, offsets and lengths are compared bit for bit where they are copies.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_bf16_rounding_of, assert_close, entries_f64, layer, log, weights, y_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


def run_prefill(torch, L, lens_t, seed, caps=None, fill_byte=None):
    B = len(lens_t)
    q_start = np.concatenate([[0], np.cumsum(lens_t)]).astype(np.int32)
    xbits = synth.make_hidden(int(q_start[-1]), seed=seed)
    cache = binding.Cache(L, caps if caps is not None else lens_t, fill_byte=fill_byte)
    y = L.prefill(cache, np.arange(B), q_start, binding.bf16_tensor(xbits))
    torch.cuda.synchronize()
    return cache, q_start, xbits, y


@pytest.mark.parametrize("lens_t", [[64], [200], [77, 130, 1], [24], [20, 13]])
def test_prefill_matches_oracle(torch_cuda, lens_t):
    log(f"prefill lens={lens_t}")
    L = layer()
    _, w64 = weights()
    cache, q_start, xbits, y = run_prefill(torch_cuda, L, lens_t, seed=1000 + sum(lens_t))
    yg = y_of(y)
    x64 = synth.bf16_bits_to_f64(xbits)
    for b, t in enumerate(lens_t):
        rows = slice(q_start[b], q_start[b + 1])
        ref = omla.forward(x64[rows], w64)
        assert_close(yg[rows], ref["y"], f"seq {b} (T={t}) y")
        c_gpu, k_gpu = entries_f64(cache.slots(b).cpu().numpy())
        assert_bf16_rounding_of(c_gpu, ref["c_hat"], f"seq {b} cached c_hat")
        assert_bf16_rounding_of(k_gpu, ref["k_pe"], f"seq {b} cached k_pe")
    assert list(cache.len_h) == list(lens_t)
    assert list(cache.len_d.cpu().numpy()) == list(lens_t)


def test_chunked_prefill_onto_cached_prefix(torch_cuda):
    """A second prefill call continues the sequence at position len (causal over prefix+new)."""
    log("chunked prefill 100 + 60")
    L = layer()
    _, w64 = weights()
    xbits = synth.make_hidden(160, seed=1234)
    cache = binding.Cache(L, [160])
    x_all = binding.bf16_tensor(xbits)
    L.prefill(cache, [0], [0, 100], x_all[:100])
    y2 = L.prefill(cache, [0], [0, 60], x_all[100:].contiguous())
    torch_cuda.cuda.synchronize()
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w64, rows=np.arange(100, 160))
    assert_close(y_of(y2), ref["y"], "second chunk y")
    assert cache.len_h[0] == 160 and int(cache.len_d[0]) == 160


def test_decode_matches_oracle_position_1000(torch_cuda):
    """One new token at position 1000 over 1000 cached positions (entries from the oracle kv path)."""
    log("decode B=1 at position 1000")
    L = layer()
    _, w64 = weights()
    x_prev = synth.bf16_bits_to_f64(synth.make_hidden(1000, seed=1001))
    c, k = omla.kv_entries(x_prev, w64)
    ent_bits = synth.f32_to_bf16_bits(np.concatenate([c, k], axis=1).astype(np.float32))
    cache = binding.Cache(L, [1001])
    L.cache_append(cache, 0, binding.bf16_tensor(ent_bits))
    xn = synth.make_hidden(1, seed=1002)
    y = L.decode(cache, [0], binding.bf16_tensor(xn))
    torch_cuda.cuda.synchronize()
    ents = synth.bf16_bits_to_f64(ent_bits)
    ref = omla.forward(synth.bf16_bits_to_f64(xn), w64, cache=(ents[:, :512], ents[:, 512:]))
    assert_close(y_of(y), ref["y"], "decode y")
    assert cache.len_h[0] == 1001 and int(cache.len_d[0]) == 1001
    # the appended entry (position 1000) is the oracle's entry within bf16 rounding
    c_gpu, k_gpu = entries_f64(cache.slots(0)[1000:].cpu().numpy())
    assert_bf16_rounding_of(c_gpu, ref["c_hat"], "new entry c_hat")
    assert_bf16_rounding_of(k_gpu, ref["k_pe"], "new entry k_pe")


def test_decode_varlen_batch(torch_cuda):
    """Batched decode over ragged cached lengths, including an empty cache and block edges."""
    lens = [0, 1, 63, 64, 65, 700, 2049]
    log(f"decode varlen lens={lens}")
    L = layer()
    _, w64 = weights()
    cache = binding.Cache(L, [n + 1 for n in lens])
    ents = {}
    for s, n in enumerate(lens):
        if n:
            e = synth.make_cache_entries(n, seed=3000 + s)
            ents[s] = e
            L.cache_append(cache, s, binding.bf16_tensor(e))
    order = np.array([5, 0, 6, 2, 1, 4, 3], dtype=np.int32)  # batch rows in a shuffled sequence order
    xn = synth.make_hidden(len(order), seed=1003)
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn)))
    torch_cuda.cuda.synchronize()
    for b, s in enumerate(order):
        if lens[s]:
            e = synth.bf16_bits_to_f64(ents[s])
            kw = dict(cache=(e[:, :512], e[:, 512:]))
        else:
            kw = {}
        ref = omla.forward(synth.bf16_bits_to_f64(xn[b:b + 1]), w64, **kw)
        assert_close(y[b:b + 1], ref["y"], f"seq {s} (L={lens[s]})")
    assert list(cache.len_h) == [n + 1 for n in lens]
    assert list(cache.len_d.cpu().numpy()) == [n + 1 for n in lens]


@pytest.mark.parametrize("B", [24, 40, 96])
def test_decode_mid_batch(torch_cuda, B):
    """Decode at 17..64 sequences (the LDS-ring projections, their K-split parts and reduction, the
    per-head absorb and W_UV products) and at 96 (the tile kernels for every product), cached
    lengths 0..600 in a shuffled batch order."""
    rng = np.random.default_rng(3100 + B)
    lens = [int(v) for v in rng.integers(0, 601, size=B)]
    lens[0] = 0
    log(f"decode mid batch B={B}")
    L = layer()
    _, w64 = weights()
    cache = binding.Cache(L, [n + 1 for n in lens])
    ents = {}
    for s, n in enumerate(lens):
        if n:
            ents[s] = synth.make_cache_entries(n, seed=3200 + s)
            L.cache_append(cache, s, binding.bf16_tensor(ents[s]))
    order = rng.permutation(B).astype(np.int32)
    xn = synth.make_hidden(B, seed=3300 + B)
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn)))
    torch_cuda.cuda.synchronize()
    for b, s in enumerate(order):
        kw = {}
        if lens[s]:
            e = synth.bf16_bits_to_f64(ents[s])
            kw = dict(cache=(e[:, :512], e[:, 512:]))
        ref = omla.forward(synth.bf16_bits_to_f64(xn[b:b + 1]), w64, **kw)
        assert_close(y[b:b + 1], ref["y"], f"row {b} seq {s} (L={lens[s]})")
    assert list(cache.len_h) == [n + 1 for n in lens]


@pytest.mark.parametrize("lens", [[700, 0], [64, 1, 1500], [33, 2000, 65, 129]])
def test_decode_small_batch(torch_cuda, lens):
    """Decode of two to four sequences: the launch sequences where the norms run inside the q_b
    kernel (one or two tokens) and W_UV inside the merge (up to four); the new cache entries too."""
    B = len(lens)
    log(f"decode small batch lens={lens}")
    L = layer()
    _, w64 = weights()
    cache = binding.Cache(L, [n + 1 for n in lens])
    ents = {}
    for s, n in enumerate(lens):
        if n:
            ents[s] = synth.make_cache_entries(n, seed=3100 + s)
            L.cache_append(cache, s, binding.bf16_tensor(ents[s]))
    order = np.arange(B, dtype=np.int32)[::-1].copy()  # batch rows in reverse sequence order
    xn = synth.make_hidden(B, seed=1013 + B)
    y = y_of(L.decode(cache, order, binding.bf16_tensor(xn)))
    torch_cuda.cuda.synchronize()
    for b, s in enumerate(order):
        e = synth.bf16_bits_to_f64(ents[s]) if lens[s] else np.zeros((0, 576))
        ref = omla.forward(synth.bf16_bits_to_f64(xn[b:b + 1]), w64, cache=(e[:, :512], e[:, 512:]))
        assert_close(y[b:b + 1], ref["y"], f"seq {s} (L={lens[s]})")
        c_gpu, k_gpu = entries_f64(cache.slots(s).cpu().numpy()[lens[s]:lens[s] + 1])
        assert_bf16_rounding_of(c_gpu, ref["c_hat"], f"seq {s} new c_hat")
        assert_bf16_rounding_of(k_gpu, ref["k_pe"], f"seq {s} new k_pe")
    assert list(cache.len_h) == [n + 1 for n in lens]
    assert list(cache.len_d.cpu().numpy()) == [n + 1 for n in lens]


def test_prefill_then_decode_steps(torch_cuda):
    """prefill(T) followed by decode steps equals the oracle's prefill over all tokens."""
    log("prefill 33 + 3 decode steps")
    L = layer()
    _, w64 = weights()
    xbits = synth.make_hidden(36, seed=1004)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [40])
    L.prefill(cache, [0], [0, 33], xt[:33])
    ys = [y_of(L.decode(cache, [0], xt[33 + i:34 + i].contiguous())) for i in range(3)]
    torch_cuda.cuda.synchronize()
    ref = omla.forward(synth.bf16_bits_to_f64(xbits), w64, rows=np.arange(33, 36))
    assert_close(np.concatenate(ys), ref["y"], "decode steps after prefill")


def test_cache_append_is_a_byte_copy_and_sentinels_survive(torch_cuda):
    import torch

    log("cache append byte copy + sentinels")
    L = layer()
    cache = binding.Cache(L, [10, 20], fill_byte=0xA5)
    e = synth.make_cache_entries(7, seed=5)
    L.cache_append(cache, 1, binding.bf16_tensor(e))
    # prefill 4 tokens into sequence 0
    L.prefill(cache, [0], [0, 4], binding.bf16_tensor(synth.make_hidden(4, seed=6)))
    torch.cuda.synchronize()
    raw = cache.data.cpu().numpy().reshape(-1, L.entry_bytes)
    o1 = int(cache.offset_h[1])
    assert np.array_equal(raw[o1:o1 + 7], np.ascontiguousarray(e).view(np.uint8).reshape(7, -1))
    assert np.all(raw[o1 + 7:o1 + 20] == 0xA5)  # unused slots of sequence 1
    assert np.all(raw[4:o1] == 0xA5)            # unused slots of sequence 0 and padding
    assert not np.all(raw[:4] == 0xA5)
    assert list(cache.len_h) == [4, 7] and list(cache.len_d.cpu().numpy()) == [4, 7]


def test_decode_is_deterministic(torch_cuda):
    log("determinism")
    L = layer()
    e = synth.make_cache_entries(3000, seed=7)
    xn = binding.bf16_tensor(synth.make_hidden(2, seed=8))
    outs = []
    for _ in range(2):
        cache = binding.Cache(L, [3001, 3001])
        L.cache_append(cache, 0, binding.bf16_tensor(e))
        L.cache_append(cache, 1, binding.bf16_tensor(e[:1500]))
        outs.append(binding.tensor_to_bf16_bits(L.decode(cache, [0, 1], xn)))
    assert np.array_equal(outs[0], outs[1])


def test_errors_leave_state_untouched(torch_cuda):
    import torch

    log("error paths")
    L = layer()
    cache = binding.Cache(L, [8], fill_byte=0x5A)
    x = binding.bf16_tensor(synth.make_hidden(9, seed=9))
    with pytest.raises(binding.MlaError) as ei:
        L.prefill(cache, [0], [0, 9], x)
    assert ei.value.status == 3  # capacity
    with pytest.raises(binding.MlaError) as ei:
        L.prefill(cache, [0], [0, 0], x)
    assert ei.value.status == 2  # a sequence with no new tokens
    with pytest.raises(binding.MlaError) as ei:
        L.decode(cache, [1], x[:1].contiguous())
    assert ei.value.status == 1  # unknown sequence id
    with pytest.raises(binding.MlaError) as ei:
        L.decode(cache, [0, 0], x[:2].contiguous())
    assert ei.value.status == 1  # repeated id
    torch.cuda.synchronize()
    assert cache.len_h[0] == 0 and int(cache.len_d[0]) == 0
    assert np.all(cache.data.cpu().numpy() == 0x5A)
    # max_positions is enforced even where the slots would allow more
    small = binding.Layer(L.weights, max_positions=4)
    c2 = binding.Cache(small, [16])
    with pytest.raises(binding.MlaError) as ei:
        small.prefill(c2, [0], [0, 5], x[:5].contiguous())
    assert ei.value.status == 3


def test_resume_from_snapshot_is_bit_identical(torch_cuda):
    """All layer state is the caller's cache and length arrays: snapshot them after a prefill,
    decode two steps, restore the snapshot (into the same buffers) and decode again; the outputs
    and the cache bytes match bit for bit."""
    import torch

    log("snapshot / restore / decode again")
    L = layer()
    xbits = synth.make_hidden(52, seed=1006)
    xt = binding.bf16_tensor(xbits)
    cache = binding.Cache(L, [64, 16])
    L.prefill(cache, [0, 1], [0, 40, 50], xt[:50])
    torch_cuda.cuda.synchronize()
    snap = (cache.data.clone(), cache.len_h.copy(), cache.len_d.clone())

    def two_steps():
        out = [binding.tensor_to_bf16_bits(L.decode(cache, [0, 1], xt[50:52].contiguous())) for _ in range(2)]
        torch.cuda.synchronize()
        return out, cache.data.clone()

    y1, c1 = two_steps()
    cache.data.copy_(snap[0])
    cache.len_h[:] = snap[1]
    cache.len_d.copy_(snap[2])
    y2, c2 = two_steps()
    assert all(np.array_equal(a, b) for a, b in zip(y1, y2))
    assert torch.equal(c1, c2)
    assert cache.len_h.tolist() == [42, 12]
