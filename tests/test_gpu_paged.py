"""GPU check of the paged latent cache (block tables over pages of 64 slots, pages from the
library's page allocator) against the same calls on a contiguous cache and against the float64
oracle.

The pages are handed out fragmented and interleaved (the allocator's free list is scrambled
first, and the sequences grow in turn), so each sequence's positions are scattered over
non-adjacent, out-of-order pages. Checked: outputs bit-identical to the contiguous cache's (the
same kernels on the same entries), every position's entry bit-identical at its paged slot,
pages nobody holds untouched, outputs within the parity bar of the oracle; a released
sequence's pages reused by a new one; a table entry outside the pool rejected before anything
runs. bf16 (ragged prefill, chunked prefill across page boundaries, decode steps) and FP8
(appended entries across page boundaries, decode).
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import assert_close, layer, log, weights, y_of
from test_gpu_fp8 import fp8_setup, pack_fp8_entries

pytestmark = pytest.mark.gpu

FILL = 0x5D
PAGE = 64


def scrambled_paged_cache(L, n_seqs, n_pages, seed):
    """A paged cache whose allocator hands pages out in a shuffled order."""
    pc = binding.PagedCache(L, n_seqs, n_pages, page_size=PAGE, fill_byte=FILL)
    ids = pc.pool.alloc(n_pages)
    pc.pool.free(np.random.default_rng(seed).permutation(ids))
    return pc


def assert_same_entries(pc, cc, seqs):
    for s in seqs:
        a = pc.slots(s).cpu().numpy()
        b = cc.slots(s).cpu().numpy()
        assert a.shape == b.shape and np.array_equal(a, b), f"sequence {s}: paged entries differ"


def assert_free_pages_untouched(pc):
    held = set(int(p) for s in range(pc.table_h.shape[0]) for p in pc.table_h[s, :pc.n_held[s]])
    raw = pc.data.cpu().numpy().reshape(pc.n_pages, PAGE * pc.entry_bytes)
    for p in range(pc.n_pages):
        if p not in held:
            assert np.all(raw[p] == FILL), f"page {p} is held by no sequence but was written"


def test_paged_bf16_prefill_chunk_decode_matches_contiguous_and_oracle():
    import torch

    L = layer()
    _, w64 = weights()
    lens = [130, 70, 20]
    log(f"paged bf16: prefill {lens}, chunked prefill of 100 onto sequence 0, two decode steps")
    pc = scrambled_paged_cache(L, 3, 24, seed=11)
    cc = binding.Cache(L, [260, 80, 30])
    # pages given in turn as the sequences grow: interleaved, out of order
    for s, n in ((0, 64), (1, 64), (2, 20), (0, 130), (1, 72)):
        pc.reserve(s, n)
    q_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xb = synth.make_hidden(int(q_start[-1]) + 100 + 6, seed=8500)
    x = binding.bf16_tensor(xb)
    n0 = int(q_start[-1])
    outs = {}
    for name, c in (("paged", pc), ("contiguous", cc)):
        y0 = y_of(L.prefill(c, [0, 1, 2], q_start, x[:n0]))
        if c is pc:
            pc.reserve(0, 232)
            pc.reserve(1, 72)
            pc.reserve(2, 22)
        y1 = y_of(L.prefill(c, [0], [0, 100], x[n0:n0 + 100].contiguous()))
        yd = [y_of(L.decode(c, [2, 0, 1], x[n0 + 100 + 3 * i:n0 + 103 + 3 * i].contiguous())) for i in range(2)]
        torch.cuda.synchronize()
        outs[name] = (y0, y1, yd)
    for a, b in zip(outs["paged"][:2] + tuple(outs["paged"][2]), outs["contiguous"][:2] + tuple(outs["contiguous"][2])):
        assert np.array_equal(a, b), "paged and contiguous outputs differ"
    assert list(pc.len_h) == list(cc.len_h) == [232, 72, 22]
    assert_same_entries(pc, cc, range(3))
    assert_free_pages_untouched(pc)
    assert sorted(set(pc.table_h[0, :pc.n_held[0]]) & set(pc.table_h[1, :pc.n_held[1]])) == []
    # the oracle: sequence 0 over its whole history (prefill 130, chunk 100, decode steps)
    x64 = synth.bf16_bits_to_f64(xb)
    rows0 = np.concatenate([np.arange(0, 130), np.arange(n0, n0 + 100), [n0 + 101, n0 + 104]])
    ref = omla.forward(x64[rows0], w64, rows=np.array([129, 180, 229, 230, 231]), absorbed=True)
    got = np.concatenate([outs["paged"][0][129:130], outs["paged"][1][[50, 99]], outs["paged"][2][0][1:2],
                          outs["paged"][2][1][1:2]])
    assert_close(got, ref["y"], "sequence 0 through prefill, chunk and decode")


def test_paged_release_and_reuse():
    import torch

    L = layer()
    _, w64 = weights()
    log("paged bf16: a released sequence's pages go to a new sequence")
    pc = scrambled_paged_cache(L, 2, 6, seed=12)
    xb = synth.make_hidden(200 + 150, seed=8600)
    x = binding.bf16_tensor(xb)
    pc.reserve(0, 200)
    L.prefill(pc, [0], [0, 200], x[:200])
    torch.cuda.synchronize()
    used = set(pc.table_h[0, :pc.n_held[0]].tolist())
    pc.release(0)
    assert pc.pool.available == 6
    pc.reserve(1, 150)
    assert set(pc.table_h[1, :pc.n_held[1]].tolist()) <= set(range(6))
    y = y_of(L.prefill(pc, [1], [0, 150], x[200:].contiguous()))
    torch.cuda.synchronize()
    assert set(pc.table_h[1, :pc.n_held[1]].tolist()) & used  # at least one page is reused
    ref = omla.forward(synth.bf16_bits_to_f64(xb[200:]), w64)
    assert_close(y, ref["y"], "new sequence on reused pages")
    assert int(pc.len_h[0]) == 0 and int(pc.len_h[1]) == 150


def test_paged_fp8_append_and_decode():
    import torch

    wq, w64, L = fp8_setup()
    lens = [150, 90]
    log(f"paged FP8: appended entries {lens} across page boundaries, one decode step")
    pc = scrambled_paged_cache(L, 2, 8, seed=13)
    cc = binding.Cache(L, [n + 1 for n in lens])
    lat = {}
    for s, n in enumerate(lens):
        pc.reserve(s, n + 1)
        e = synth.bf16_bits_to_f64(synth.make_cache_entries(n, seed=8700 + s))
        raw, c_dq = pack_fp8_entries(e[:, :512], e[:, 512:])
        lat[s] = (c_dq, e[:, 512:].astype(np.float32).astype(np.float64))
        t = torch.from_numpy(raw).cuda()
        L.cache_append(pc, s, t)
        L.cache_append(cc, s, t)
    xb = synth.make_hidden(2, seed=8800)
    yp = y_of(L.decode(pc, [1, 0], binding.bf16_tensor(xb)))
    yc = y_of(L.decode(cc, [1, 0], binding.bf16_tensor(xb)))
    torch.cuda.synchronize()
    assert np.array_equal(yp, yc)
    assert_same_entries(pc, cc, range(2))
    assert_free_pages_untouched(pc)
    for b, s in enumerate((1, 0)):
        ref = omla.forward(synth.bf16_bits_to_f64(xb[b:b + 1]), w64, cache=lat[s], w8a8=True)
        assert_close(yp[b:b + 1], ref["y"], f"FP8 paged seq {s}")


def test_paged_rejects_a_page_outside_the_pool():
    import torch

    L = layer()
    log("paged: a table entry outside the pool is rejected before any work")
    pc = scrambled_paged_cache(L, 1, 4, seed=14)
    pc.reserve(0, 100)
    pc.table_h[0, 1] = 9  # the host table names a page the cache does not have
    x = binding.bf16_tensor(synth.make_hidden(100, seed=8900))
    with pytest.raises(binding.MlaError) as ei:
        L.prefill(pc, [0], [0, 100], x)
    assert ei.value.status == 1
    torch.cuda.synchronize()
    assert int(pc.len_h[0]) == 0 and int(pc.len_d[0]) == 0
    assert bool((pc.data == FILL).all())
