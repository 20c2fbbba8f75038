"""The C-ABI library loads on a machine without a GPU, exports every declared symbol, and
rejects invalid arguments before touching HIP (no compute calls here)."""
import ctypes
import os
import re

import pytest

from head_latent_attention_proj_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libmla.so not built")
    return binding.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_symbols()
    assert names, "no declarations found"
    assert set(binding.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(8):
        assert L.mla_status_str(code)
    assert L.mla_status_str(0) == b"ok"


def test_config_validation_without_gpu(L):
    cfg = binding.make_config(max_positions=4096)
    assert L.mla_cache_entry_bytes(ctypes.byref(cfg)) == 1152
    assert L.mla_packed_weight_bytes(ctypes.byref(cfg)) > (2112 * 7168 + 64 * 512 * 128) * 2
    fp8 = binding.make_config(max_positions=4096, wdtype=binding.WDTYPE_FP8)
    assert L.mla_cache_entry_bytes(ctypes.byref(fp8)) == 784
    bad = binding.make_config()
    bad.heads = 32
    assert L.mla_packed_weight_bytes(ctypes.byref(bad)) == 0
    assert b"built for" in L.mla_last_error()
    bad = binding.make_config(max_positions=131073)
    assert L.mla_cache_entry_bytes(ctypes.byref(bad)) == 0
    bad = binding.make_config(wdtype=7)
    assert L.mla_cache_entry_bytes(ctypes.byref(bad)) == 0
    # YaRN RoPE: the released rope_scaling validates; a zero-filled tail (plain RoPE) too
    yarn = binding.make_config(max_positions=4096, rope_scaling=binding.KIMI_K2_YARN)
    assert L.mla_cache_entry_bytes(ctypes.byref(yarn)) == 1152
    assert yarn.rope_factor == 32.0 and yarn.rope_orig_max == 4096
    for key, val in (("original_max_position_embeddings", 0), ("beta_slow", 0.0), ("beta_fast", 0.5),
                     ("mscale", -1.0), ("factor", float("inf"))):
        bad = binding.make_config(rope_scaling={**binding.KIMI_K2_YARN, key: val})
        assert L.mla_cache_entry_bytes(ctypes.byref(bad)) == 0, key
    assert b"rope" in L.mla_last_error()
    # factor <= 1 ignores the other fields
    off = binding.make_config(rope_scaling={"factor": 1.0, "beta_slow": -3.0})
    assert L.mla_cache_entry_bytes(ctypes.byref(off)) == 1152


def test_init_rejects_null_and_unsupported_before_any_hip_call(L):
    ctx = ctypes.c_void_p()
    w = binding.MlaWeights()
    cfg = binding.make_config(max_positions=64)
    assert L.mla_init_weights(ctypes.byref(cfg), ctypes.byref(w), None, 0, None, ctypes.byref(ctx)) == 1
    assert not ctx.value
    bad = binding.make_config()
    bad.hidden = 4096
    assert L.mla_init_weights(ctypes.byref(bad), ctypes.byref(w), None, 0, None, ctypes.byref(ctx)) == 4
    # misaligned weight pointers are rejected before use (the addresses are never dereferenced)
    for i, name in enumerate(("q_a", "q_a_norm", "q_b", "kv_a", "kv_a_norm", "kv_b", "o")):
        setattr(w, name, 0x1000 * (i + 1) + 2)
    assert L.mla_init_weights(ctypes.byref(cfg), ctypes.byref(w), 0x100000, 1 << 30, None, ctypes.byref(ctx)) == 7


def test_calls_reject_null_context(L):
    desc = binding.MlaCacheDesc()
    assert L.mla_prefill(None, ctypes.byref(desc), None, None, None, None, 1, None, None, None, 0, None) == 1
    assert L.mla_decode(None, ctypes.byref(desc), None, None, 1, None, None, None, 0, None) == 1
    assert L.mla_cache_append(None, ctypes.byref(desc), 0, None, 1, None) == 1
    assert L.mla_block_prefill(None, ctypes.byref(desc), None, None, None, None, 1, None, None, None, None, 0,
                               None) == 1
    assert L.mla_block_decode(None, ctypes.byref(desc), None, None, 1, None, None, None, None, 0, None) == 1
    assert L.mla_block_prefill_workspace_bytes(None, 1, 1, 1) == 0
    assert L.mla_block_decode_workspace_bytes(None, 1, 1) == 0
    assert L.mla_prefill_workspace_bytes(None, 1, 1, 1) == 0
    assert L.mla_decode_workspace_bytes(None, 1, 1) == 0
    # more than 4096 sequences in one call: rejected before anything else is looked at
    assert L.mla_decode(None, ctypes.byref(desc), None, None, 4097, None, None, None, 0, None) == 4
    assert L.mla_prefill(None, ctypes.byref(desc), None, None, None, None, 4097, None, None, None, 0, None) == 4
    L.mla_destroy(None)


def test_cache_pool_plan_matches_page_bytes(L):
    """A 61-layer pool costs 70,272 B per position in bf16, the latent cache figure printed on the
    dense-block attention page ("In numbers", tests/golden/page_facts.json), and 61 x 784 in the FP8
    slot format; offsets are aligned runs per sequence."""
    import json

    import numpy as np

    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))["cache_bytes_per_token_61_layers"]
    n = facts["layers"]
    for wdtype, per_layer in ((binding.WDTYPE_BF16, facts["latent_bf16"] // n), (binding.WDTYPE_FP8, 784)):
        cfg = binding.make_config(wdtype=wdtype)
        caps = np.array([1], dtype=np.int32)
        off = np.zeros(1, dtype=np.int64)
        total, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
        assert L.mla_cache_pool_plan(ctypes.byref(cfg), n, 1, caps.ctypes.data, 1, off.ctypes.data,
                                     ctypes.byref(total), ctypes.byref(lb), ctypes.byref(pb)) == 0
        assert (total.value, lb.value, pb.value) == (1, per_layer, n * per_layer)
    assert n * 1152 == facts["latent_bf16"]
    cfg = binding.make_config()
    caps = np.array([5, 0, 17, 16], dtype=np.int32)
    off = np.zeros(4, dtype=np.int64)
    total, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.mla_cache_pool_plan(ctypes.byref(cfg), 3, 4, caps.ctypes.data, 16, off.ctypes.data,
                                 ctypes.byref(total), ctypes.byref(lb), ctypes.byref(pb)) == 0
    assert off.tolist() == [0, 16, 16, 48] and total.value == 64
    assert lb.value == 64 * 1152 and pb.value == 3 * 64 * 1152


def test_cache_pool_rejects_bad_arguments(L):
    import numpy as np

    cfg = binding.make_config(max_positions=4096)
    off = np.zeros(2, dtype=np.int64)
    total, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
    args = lambda caps, n_layers=2, align=16: (ctypes.byref(cfg), n_layers, len(caps), caps.ctypes.data, align,
                                              off.ctypes.data, ctypes.byref(total), ctypes.byref(lb), ctypes.byref(pb))
    assert L.mla_cache_pool_plan(*args(np.array([8, 5000], dtype=np.int32))) == 3  # MLA_E_CAPACITY
    assert L.mla_cache_pool_plan(*args(np.array([8, -1], dtype=np.int32))) == 1
    assert L.mla_cache_pool_plan(*args(np.array([0, 0], dtype=np.int32))) == 1
    assert L.mla_cache_pool_plan(*args(np.array([8, 8], dtype=np.int32), n_layers=0)) == 1
    assert L.mla_cache_pool_plan(*args(np.array([8, 8], dtype=np.int32), align=0)) == 1
    desc = binding.MlaCacheDesc()
    buf = ctypes.create_string_buffer(4096 + 16)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    assert L.mla_cache_pool_layer(ctypes.c_void_p(base), 4096, 1152, 3, ctypes.byref(desc)) == 1  # past the end
    assert L.mla_cache_pool_layer(ctypes.c_void_p(base), 4096, 1000, 0, ctypes.byref(desc)) == 7  # MLA_E_ALIGN
    assert L.mla_cache_pool_layer(ctypes.c_void_p(base), 4096, 1152, 2, None) == 1
    assert L.mla_cache_pool_layer(ctypes.c_void_p(base), 4096, 1152, 1, ctypes.byref(desc)) == 0
    assert desc.data == base + 1152


def test_page_pool_hands_out_and_takes_back_pages(L):
    """The host page allocator of paged caches: ids in order, FIFO reuse of released pages, and
    refusals (too few free, double free, foreign id) that change nothing."""
    import numpy as np

    pool = binding.PagePool(5)
    assert pool.available == 5
    assert pool.alloc(3).tolist() == [0, 1, 2] and pool.available == 2
    with pytest.raises(binding.MlaError) as ei:
        pool.alloc(3)
    assert ei.value.status == 3 and pool.available == 2  # MLA_E_CAPACITY, nothing taken
    pool.free([1])
    assert pool.available == 3
    assert pool.alloc(3).tolist() == [3, 4, 1]  # never-used pages first, then the released one
    with pytest.raises(binding.MlaError) as ei:
        pool.free([2, 2])
    assert ei.value.status == 1 and pool.available == 0  # a double free is refused as a whole
    with pytest.raises(binding.MlaError):
        pool.free([7])
    pool.free([2, 0])
    assert pool.available == 2 and pool.alloc(2).tolist() == [2, 0]
    h = ctypes.c_void_p()
    assert L.mla_page_pool_create(0, ctypes.byref(h)) == 1
    assert L.mla_page_pool_available(None) == -1
    ids = np.zeros(1, dtype=np.int32)
    assert L.mla_page_pool_alloc(None, 1, ids.ctypes.data) == 1
