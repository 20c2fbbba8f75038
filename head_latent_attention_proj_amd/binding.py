"""Thin ctypes binding over libmla.so (include/mla.h). Argument marshalling only.

torch provides device memory and the stream; every step of the layer runs in the library's HIP
kernels. Loading fails loudly if the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_E_ARG", 2: "MLA_E_SHAPE", 3: "MLA_E_CAPACITY", 4: "MLA_E_UNSUPPORTED",
                5: "MLA_E_WORKSPACE", 6: "MLA_E_HIP", 7: "MLA_E_ALIGN"}
WDTYPE_BF16 = 0
WDTYPE_FP8 = 1

EXPORTED = (
    "mla_packed_weight_bytes", "mla_cache_entry_bytes", "mla_prefill_workspace_bytes",
    "mla_decode_workspace_bytes", "mla_init_weights", "mla_prefill", "mla_decode",
    "mla_cache_append", "mla_destroy", "mla_status_str", "mla_last_error",
    "mla_block_prefill_workspace_bytes", "mla_block_decode_workspace_bytes", "mla_block_prefill", "mla_block_decode",
    "mla_cache_pool_plan", "mla_cache_pool_layer",
    "mla_test_gemm_workspace_bytes", "mla_test_gemm", "mla_decode_static", "mla_test_probe_stage",
    "mla_page_pool_create", "mla_page_pool_alloc", "mla_page_pool_free", "mla_page_pool_available",
    "mla_page_pool_destroy", "mla_test_gemm_fp8_workspace_bytes", "mla_test_gemm_fp8",
)
STAGE = {"none": 0, "qkva": 1, "qb": 2, "kvb": 3, "oproj": 4, "absorb": 5, "uv": 6, "decode_attn": 7,
         "prefill_attn": 8}


class MlaConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("q_lora", ctypes.c_int32), ("kv_lora", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("qk_nope", ctypes.c_int32), ("qk_rope", ctypes.c_int32),
                ("v_head", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("max_positions", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("rope_factor", ctypes.c_float), ("rope_orig_max", ctypes.c_int32), ("rope_beta_fast", ctypes.c_float),
                ("rope_beta_slow", ctypes.c_float), ("rope_mscale", ctypes.c_float), ("rope_mscale_all_dim", ctypes.c_float)]


class MlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q_a", "q_a_norm", "q_b", "kv_a", "kv_a_norm", "kv_b", "o")] + \
               [(n, ctypes.c_void_p) for n in ("q_a_s", "q_b_s", "kv_a_s", "kv_b_s", "o_s")]


class MlaCacheDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("offset_h", ctypes.c_void_p), ("offset_d", ctypes.c_void_p),
                ("len_h", ctypes.c_void_p), ("len_d", ctypes.c_void_p), ("cap_h", ctypes.c_void_p),
                ("n_seqs", ctypes.c_int32), ("total_slots", ctypes.c_int64),
                ("block_table_h", ctypes.c_void_p), ("block_table_d", ctypes.c_void_p),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


class MlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla.so (built by head_latent_attention_proj_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m head_latent_attention_proj_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.mla_packed_weight_bytes.argtypes = [ctypes.POINTER(MlaConfig)]
    L.mla_packed_weight_bytes.restype = sz
    L.mla_cache_entry_bytes.argtypes = [ctypes.POINTER(MlaConfig)]
    L.mla_cache_entry_bytes.restype = sz
    L.mla_prefill_workspace_bytes.argtypes = [vp, i32, i32, i64]
    L.mla_prefill_workspace_bytes.restype = sz
    L.mla_decode_workspace_bytes.argtypes = [vp, i32, i64]
    L.mla_decode_workspace_bytes.restype = sz
    L.mla_init_weights.argtypes = [ctypes.POINTER(MlaConfig), ctypes.POINTER(MlaWeights), vp, sz, vp,
                                   ctypes.POINTER(vp)]
    L.mla_init_weights.restype = ctypes.c_int
    L.mla_prefill.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.mla_prefill.restype = ctypes.c_int
    L.mla_decode.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), vp, vp, i32, vp, vp, vp, sz, vp]
    L.mla_decode.restype = ctypes.c_int
    L.mla_decode_static.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), vp, vp, i32, vp, vp, vp]
    L.mla_decode_static.restype = ctypes.c_int
    L.mla_block_prefill_workspace_bytes.argtypes = [vp, i32, i32, i64]
    L.mla_block_prefill_workspace_bytes.restype = sz
    L.mla_block_decode_workspace_bytes.argtypes = [vp, i32, i64]
    L.mla_block_decode_workspace_bytes.restype = sz
    L.mla_block_prefill.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.mla_block_prefill.restype = ctypes.c_int
    L.mla_block_decode.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.mla_block_decode.restype = ctypes.c_int
    L.mla_cache_pool_plan.argtypes = [ctypes.POINTER(MlaConfig), i32, i32, vp, i32, vp, ctypes.POINTER(i64),
                                      ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.mla_cache_pool_plan.restype = ctypes.c_int
    L.mla_cache_pool_layer.argtypes = [vp, sz, sz, i32, ctypes.POINTER(MlaCacheDesc)]
    L.mla_cache_pool_layer.restype = ctypes.c_int
    L.mla_cache_append.argtypes = [vp, ctypes.POINTER(MlaCacheDesc), i32, vp, i32, vp]
    L.mla_cache_append.restype = ctypes.c_int
    L.mla_destroy.argtypes = [vp]
    L.mla_destroy.restype = None
    L.mla_status_str.argtypes = [ctypes.c_int]
    L.mla_status_str.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_test_gemm_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.mla_test_gemm_workspace_bytes.restype = sz
    L.mla_test_gemm.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, vp, i64, i64, i32, i32, vp, sz, vp]
    L.mla_test_gemm.restype = ctypes.c_int
    L.mla_test_gemm_fp8_workspace_bytes.argtypes = [i32, i32, i32]
    L.mla_test_gemm_fp8_workspace_bytes.restype = sz
    L.mla_test_gemm_fp8.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.mla_test_gemm_fp8.restype = ctypes.c_int
    L.mla_test_probe_stage.argtypes = [i32, vp, vp]
    L.mla_test_probe_stage.restype = ctypes.c_int
    L.mla_page_pool_create.argtypes = [i32, ctypes.POINTER(vp)]
    L.mla_page_pool_create.restype = ctypes.c_int
    L.mla_page_pool_alloc.argtypes = [vp, i32, vp]
    L.mla_page_pool_alloc.restype = ctypes.c_int
    L.mla_page_pool_free.argtypes = [vp, vp, i32]
    L.mla_page_pool_free.restype = ctypes.c_int
    L.mla_page_pool_available.argtypes = [vp]
    L.mla_page_pool_available.restype = i32
    L.mla_page_pool_destroy.argtypes = [vp]
    L.mla_page_pool_destroy.restype = None
    _lib = L
    return L


def check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, lib().mla_last_error().decode())


# rope_scaling of the released configuration (config excerpt on the "KV cache" page)
KIMI_K2_YARN = {"factor": 32.0, "original_max_position_embeddings": 4096, "beta_fast": 1.0, "beta_slow": 1.0,
                "mscale": 1.0, "mscale_all_dim": 1.0}


def make_config(max_positions: int = 131072, wdtype: int = WDTYPE_BF16, softmax_scale: float = 0.0,
                eps: float = 1e-6, theta: float = 50000.0, rope_scaling: dict | None = None) -> MlaConfig:
    """Layer config; rope_scaling (keys as in the config excerpt's rope_scaling) selects YaRN RoPE."""
    y = rope_scaling or {}
    return MlaConfig(7168, 1536, 512, 64, 128, 64, 128, eps, theta, softmax_scale, max_positions, wdtype,
                     float(y.get("factor", 0.0)), int(y.get("original_max_position_embeddings", 0)),
                     float(y.get("beta_fast", 0.0)), float(y.get("beta_slow", 0.0)),
                     float(y.get("mscale", 0.0)), float(y.get("mscale_all_dim", 0.0)))


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


class Cache:
    """Caller-owned latent cache: device slots plus host/device offset and length arrays."""

    def __init__(self, layer: "Layer", caps, device="cuda", fill_byte: int | None = None, align: int = 16):
        import torch

        caps = np.asarray(caps, dtype=np.int64)
        rounded = ((caps + align - 1) // align) * align
        self.offset_h = np.zeros(len(caps), dtype=np.int64)
        if len(caps) > 1:
            self.offset_h[1:] = np.cumsum(rounded)[:-1]
        self.cap_h = caps.astype(np.int32)
        self.len_h = np.zeros(len(caps), dtype=np.int32)
        self.total_slots = int(rounded.sum())
        self.entry_bytes = layer.entry_bytes
        self.data = torch.empty(self.total_slots * self.entry_bytes, dtype=torch.uint8, device=device)
        if fill_byte is not None:
            self.data.fill_(fill_byte)
        self.offset_d = torch.from_numpy(self.offset_h).to(device)
        self.len_d = torch.zeros(len(caps), dtype=torch.int32, device=device)
        self._desc = MlaCacheDesc(self.data.data_ptr(), self.offset_h.ctypes.data, self.offset_d.data_ptr(),
                                  self.len_h.ctypes.data, self.len_d.data_ptr(), self.cap_h.ctypes.data,
                                  len(caps), self.total_slots, None, None, 0, 0)

    @property
    def desc(self) -> MlaCacheDesc:
        return self._desc

    def held(self, seq: int) -> int:
        """Positions held by `seq` (0 for an id outside the cache: the library rejects it)."""
        return int(self.len_h[seq]) if 0 <= seq < len(self.len_h) else 0

    def slots(self, seq: int):
        """View of sequence `seq`'s used slots as [len, entry_bytes] uint8."""
        o, n = int(self.offset_h[seq]), int(self.len_h[seq])
        return self.data.view(-1, self.entry_bytes)[o:o + n]


class PagePool:
    """The library's host page allocator (mla_page_pool_*): page ids 0 .. n_pages-1, handed out and
    taken back; released pages are reused oldest first."""

    def __init__(self, n_pages: int):
        h = ctypes.c_void_p()
        check(lib().mla_page_pool_create(n_pages, ctypes.byref(h)))
        self._h = h
        self.n_pages = n_pages

    def alloc(self, n: int) -> np.ndarray:
        ids = np.empty(max(n, 1), dtype=np.int32)
        check(lib().mla_page_pool_alloc(self._h, n, ids.ctypes.data))
        return ids[:n]

    def free(self, ids) -> None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        check(lib().mla_page_pool_free(self._h, ids.ctypes.data, len(ids)))

    @property
    def available(self) -> int:
        return lib().mla_page_pool_available(self._h)

    def __del__(self):
        try:
            if self._h:
                lib().mla_page_pool_destroy(self._h)
                self._h = None
        except Exception:
            pass


class PagedCache(Cache):
    """Paged latent cache: n_pages pages of page_size slots in one device buffer, a block table per
    sequence (host + device copy) and pages taken from a PagePool as sequences grow (`reserve`) and
    given back when a sequence ends (`release`). Same interface as Cache for the layer calls."""

    def __init__(self, layer: "Layer", n_seqs: int, n_pages: int, page_size: int = 64, max_pages: int | None = None,
                 pool: PagePool | None = None, device="cuda", fill_byte: int | None = None):
        import torch

        self.page_size, self.n_pages = page_size, n_pages
        self.max_pages = max_pages or n_pages
        self.pool = pool or PagePool(n_pages)
        self.entry_bytes = layer.entry_bytes
        self.total_slots = n_pages * page_size
        self.data = torch.empty(self.total_slots * self.entry_bytes, dtype=torch.uint8, device=device)
        if fill_byte is not None:
            self.data.fill_(fill_byte)
        self.table_h = np.full((n_seqs, self.max_pages), -1, dtype=np.int32)
        self.table_d = torch.from_numpy(self.table_h).to(device)
        self.n_held = np.zeros(n_seqs, dtype=np.int32)  # pages held per sequence
        self.cap_h = np.zeros(n_seqs, dtype=np.int32)
        self.len_h = np.zeros(n_seqs, dtype=np.int32)
        self.len_d = torch.zeros(n_seqs, dtype=torch.int32, device=device)
        self.offset_h = None
        self._desc = MlaCacheDesc(self.data.data_ptr(), None, None, self.len_h.ctypes.data, self.len_d.data_ptr(),
                                  self.cap_h.ctypes.data, n_seqs, self.total_slots, self.table_h.ctypes.data,
                                  self.table_d.data_ptr(), page_size, self.max_pages)

    def reserve(self, seq: int, positions: int) -> None:
        """Give sequence `seq` pages for `positions` positions in all (its capacity)."""
        need = -(-positions // self.page_size)
        if need > self.n_held[seq]:
            ids = self.pool.alloc(int(need - self.n_held[seq]))
            self.table_h[seq, self.n_held[seq]:need] = ids
            self.n_held[seq] = need
            self.table_d[seq].copy_(torch_from(self.table_h[seq]))
        self.cap_h[seq] = max(int(self.cap_h[seq]), positions)

    def release(self, seq: int) -> None:
        """Give the sequence's pages back to the pool and empty it."""
        import torch

        if self.n_held[seq]:
            self.pool.free(self.table_h[seq, :self.n_held[seq]])
        self.table_h[seq, :] = -1
        self.table_d[seq].copy_(torch_from(self.table_h[seq]))
        self.n_held[seq] = 0
        self.cap_h[seq] = 0
        self.len_h[seq] = 0
        self.len_d[seq] = 0
        torch.cuda.synchronize()

    def slot_index(self, seq: int, positions) -> np.ndarray:
        p = np.asarray(positions, dtype=np.int64)
        return self.table_h[seq, p // self.page_size].astype(np.int64) * self.page_size + p % self.page_size

    def slots(self, seq: int):
        """Sequence `seq`'s used slots in position order as [len, entry_bytes] uint8 (a gathered copy)."""
        import torch

        idx = torch.from_numpy(self.slot_index(seq, np.arange(int(self.len_h[seq])))).to(self.data.device)
        return self.data.view(-1, self.entry_bytes)[idx]


def torch_from(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a))


class CachePool:
    """One device buffer holding the latent caches of a stack of layers (mla_cache_pool_plan): every
    layer shares the slot layout (offsets, capacities); each layer keeps its own lengths.
    `layer(l)` is layer l's cache, used like a Cache."""

    def __init__(self, cfg: MlaConfig, n_layers: int, caps, align: int = 16, device="cuda", fill_byte: int | None = None):
        import torch

        caps = np.ascontiguousarray(caps, dtype=np.int32)
        self.cap_h = caps
        self.offset_h = np.zeros(len(caps), dtype=np.int64)
        total, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
        check(lib().mla_cache_pool_plan(ctypes.byref(cfg), n_layers, len(caps), caps.ctypes.data, align,
                                        self.offset_h.ctypes.data, ctypes.byref(total), ctypes.byref(lb),
                                        ctypes.byref(pb)))
        self.total_slots, self.layer_bytes, self.pool_bytes = total.value, lb.value, pb.value
        self.entry_bytes = lib().mla_cache_entry_bytes(ctypes.byref(cfg))
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=device)
        if fill_byte is not None:
            self.pool.fill_(fill_byte)
        self.offset_d = torch.from_numpy(self.offset_h).to(device)
        self._layers = [_PoolLayerCache(self, l, device) for l in range(n_layers)]

    def layer(self, l: int) -> "Cache":
        return self._layers[l]


class _PoolLayerCache(Cache):
    """Layer l's view of a CachePool (same interface as Cache)."""

    def __init__(self, pool: CachePool, l: int, device):
        import torch

        self.offset_h, self.offset_d, self.cap_h = pool.offset_h, pool.offset_d, pool.cap_h
        self.len_h = np.zeros(len(pool.cap_h), dtype=np.int32)
        self.len_d = torch.zeros(len(pool.cap_h), dtype=torch.int32, device=device)
        self.total_slots, self.entry_bytes = pool.total_slots, pool.entry_bytes
        self._desc = MlaCacheDesc(None, self.offset_h.ctypes.data, self.offset_d.data_ptr(), self.len_h.ctypes.data,
                                  self.len_d.data_ptr(), self.cap_h.ctypes.data, len(pool.cap_h), pool.total_slots,
                                  None, None, 0, 0)
        check(lib().mla_cache_pool_layer(_ptr(pool.pool), pool.pool_bytes, pool.layer_bytes, l, ctypes.byref(self._desc)))
        self.data = pool.pool[l * pool.layer_bytes:(l + 1) * pool.layer_bytes]


class Layer:
    """One MLA layer: a library context over caller-owned (torch) weights."""

    def __init__(self, weights: dict, max_positions: int = 131072, wdtype: int = WDTYPE_BF16, stream=None,
                 rope_scaling: dict | None = None, softmax_scale: float = 0.0):
        import torch

        L = lib()
        self.cfg = make_config(max_positions, wdtype, softmax_scale=softmax_scale, rope_scaling=rope_scaling)
        self.weights = weights  # keep the referenced tensors alive
        w = MlaWeights()
        for name in ("q_a", "q_a_norm", "q_b", "kv_a", "kv_a_norm", "kv_b", "o"):
            setattr(w, name, weights[name].data_ptr())
        if wdtype == WDTYPE_FP8:
            for name in ("q_a", "q_b", "kv_a", "kv_b", "o"):
                setattr(w, name + "_s", weights[name + "_s"].data_ptr())
        nbytes = L.mla_packed_weight_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            raise MlaError(1, L.mla_last_error().decode())
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ctx = ctypes.c_void_p()
        check(L.mla_init_weights(ctypes.byref(self.cfg), ctypes.byref(w), _ptr(self.packed), nbytes,
                                 _stream(stream), ctypes.byref(ctx)))
        self.ctx = ctx
        self.entry_bytes = L.mla_cache_entry_bytes(ctypes.byref(self.cfg))
        self._ws = None

    def close(self):
        if self.ctx:
            lib().mla_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, nbytes: int, stream=None):
        import torch

        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        return self._ws

    def prefill_workspace_bytes(self, max_tokens: int, max_batch: int, max_keys: int) -> int:
        return lib().mla_prefill_workspace_bytes(self.ctx, max_tokens, max_batch, max_keys)

    def decode_workspace_bytes(self, max_batch: int, max_keys: int) -> int:
        return lib().mla_decode_workspace_bytes(self.ctx, max_batch, max_keys)

    def prefill(self, cache: Cache, seq_ids, q_start, x, y=None, seq_ids_d=None, q_start_d=None, stream=None):
        """x: [sum T, 7168] bf16 cuda; q_start: B+1 row offsets. Returns y [sum T, 7168] bf16.
        seq_ids_d / q_start_d: optional device copies of seq_ids / q_start (int32), made here if absent."""
        import torch

        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        q_start = np.ascontiguousarray(q_start, dtype=np.int32)
        B = len(seq_ids)
        keys = int(sum(cache.held(s) + int(q_start[b + 1] - q_start[b]) for b, s in enumerate(seq_ids)))
        ws = self.workspace(self.prefill_workspace_bytes(int(q_start[-1]), B, keys), stream)
        if y is None:
            y = torch.empty_like(x)
        sid_d = seq_ids_d if seq_ids_d is not None else torch.from_numpy(seq_ids).to(x.device)
        qs_d = q_start_d if q_start_d is not None else torch.from_numpy(q_start).to(x.device)
        check(lib().mla_prefill(self.ctx, ctypes.byref(cache.desc), seq_ids.ctypes.data, _ptr(sid_d),
                                q_start.ctypes.data, _ptr(qs_d), B, _ptr(x), _ptr(y), _ptr(ws), ws.numel(),
                                _stream(stream)))
        self._keep = (sid_d, qs_d)  # device copies stay alive until the next call
        return y

    def decode(self, cache: Cache, seq_ids, x, y=None, seq_ids_d=None, stream=None):
        """One new token per sequence: x [B, 7168] bf16 cuda. Returns y [B, 7168] bf16."""
        import torch

        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        B = len(seq_ids)
        keys = int(sum(cache.held(s) + 1 for s in seq_ids))
        ws = self.workspace(self.decode_workspace_bytes(B, keys), stream)
        if y is None:
            y = torch.empty_like(x)
        if seq_ids_d is None:
            seq_ids_d = torch.from_numpy(seq_ids).to(x.device)
        check(lib().mla_decode(self.ctx, ctypes.byref(cache.desc), seq_ids.ctypes.data, _ptr(seq_ids_d), B,
                               _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
        self._keep = (seq_ids_d,)
        return y

    def decode_static(self, cache: Cache, seq_ids, x, y=None, seq_ids_d=None, stream=None):
        """mla_decode_static: the same step as decode() on the library's own static scratch (no
        workspace, nothing allocated by the call itself). Returns y [B, 7168] bf16."""
        import torch

        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        B = len(seq_ids)
        if y is None:
            y = torch.empty_like(x)
        if seq_ids_d is None:
            seq_ids_d = torch.from_numpy(seq_ids).to(x.device)
        check(lib().mla_decode_static(self.ctx, ctypes.byref(cache.desc), seq_ids.ctypes.data, _ptr(seq_ids_d), B,
                                      _ptr(x), _ptr(y), _stream(stream)))
        self._keep = (seq_ids_d,)
        return y

    def block_prefill(self, cache: Cache, seq_ids, q_start, norm_weight, x, h=None, stream=None):
        """Attention half of a decoder block, h = x + MLA(RMSNorm(x)); x [sum T, 7168] bf16 cuda,
        norm_weight [7168] bf16 cuda. h may be x (in place). Returns h."""
        import torch

        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        q_start = np.ascontiguousarray(q_start, dtype=np.int32)
        B = len(seq_ids)
        keys = int(sum(cache.held(s) + int(q_start[b + 1] - q_start[b]) for b, s in enumerate(seq_ids)))
        ws = self.workspace(lib().mla_block_prefill_workspace_bytes(self.ctx, int(q_start[-1]), B, keys), stream)
        if h is None:
            h = torch.empty_like(x)
        sid_d = torch.from_numpy(seq_ids).to(x.device)
        qs_d = torch.from_numpy(q_start).to(x.device)
        check(lib().mla_block_prefill(self.ctx, ctypes.byref(cache.desc), seq_ids.ctypes.data, _ptr(sid_d),
                                      q_start.ctypes.data, _ptr(qs_d), B, _ptr(norm_weight), _ptr(x), _ptr(h),
                                      _ptr(ws), ws.numel(), _stream(stream)))
        self._keep = (sid_d, qs_d)
        return h

    def block_decode(self, cache: Cache, seq_ids, norm_weight, x, h=None, seq_ids_d=None, stream=None):
        """Decode step of the block's attention half: x [B, 7168] bf16 cuda. Returns h."""
        import torch

        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        B = len(seq_ids)
        keys = int(sum(cache.held(s) + 1 for s in seq_ids))
        ws = self.workspace(lib().mla_block_decode_workspace_bytes(self.ctx, B, keys), stream)
        if h is None:
            h = torch.empty_like(x)
        if seq_ids_d is None:
            seq_ids_d = torch.from_numpy(seq_ids).to(x.device)
        check(lib().mla_block_decode(self.ctx, ctypes.byref(cache.desc), seq_ids.ctypes.data, _ptr(seq_ids_d), B,
                                     _ptr(norm_weight), _ptr(x), _ptr(h), _ptr(ws), ws.numel(), _stream(stream)))
        self._keep = (seq_ids_d,)
        return h

    def cache_append(self, cache: Cache, seq: int, entries, stream=None):
        """entries: cuda tensor holding n * entry_bytes bytes in the slot format."""
        n = entries.numel() * entries.element_size() // self.entry_bytes
        check(lib().mla_cache_append(self.ctx, ctypes.byref(cache.desc), seq, _ptr(entries), n, _stream(stream)))


def probe_stage(stage: str, ev_before, ev_after) -> None:
    """Arm mla_test_probe_stage for the next layer call on this thread: the two torch.cuda.Event
    objects (each recorded once before, so that they exist) are recorded around `stage`."""
    check(lib().mla_test_probe_stage(STAGE[stage], ctypes.c_void_p(ev_before.cuda_event),
                                     ctypes.c_void_p(ev_after.cuda_event)))


def weights_to_device(wbits: dict, device="cuda") -> dict:
    """numpy bf16 bits / e4m3 codes / float32 scales -> torch tensors on the device."""
    import torch

    out = {}
    for k, v in wbits.items():
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return out


def bf16_tensor(bits: np.ndarray, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def tensor_to_bf16_bits(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


class Gemm:
    """The library's projection kernel on its own (mla_test_gemm): C = A B^T per batch."""

    def __init__(self):
        self._ws = None

    def __call__(self, A, B, C, M, N, K, batch=1, lda=None, ldb=None, ldc=None, sA=0, sB=0, sC=0,
                 stage="none", stream=None):
        import torch

        need = lib().mla_test_gemm_workspace_bytes(M, N, K, batch)
        if need == 0:
            raise MlaError(1, "invalid GEMM shape")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=A.device)
        out_bf16 = 1 if C.dtype == torch.bfloat16 else 0
        check(lib().mla_test_gemm(M, N, K, batch, _ptr(A), lda or K, sA, _ptr(B), ldb or K, sB, _ptr(C),
                                  ldc or N, sC, out_bf16, STAGE[stage], _ptr(self._ws), self._ws.numel(),
                                  _stream(stream)))
        return C

    def fp8(self, A, a_scale, B, b_scale, C, M, N, K, precise: bool, stream=None):
        """mla_test_gemm_fp8: C [M, N] float32 = dequant(A) dequant(B)^T from E4M3FN codes (uint8
        tensors [M, K], [N, K]) and float32 scales [M, K/128], [ceil(N/128), K/128]."""
        import torch

        need = lib().mla_test_gemm_fp8_workspace_bytes(M, N, K)
        if need == 0:
            raise MlaError(1, "invalid GEMM shape")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=A.device)
        check(lib().mla_test_gemm_fp8(M, N, K, _ptr(A), _ptr(a_scale), _ptr(B), _ptr(b_scale), _ptr(C),
                                      1 if precise else 0, _ptr(self._ws), self._ws.numel(), _stream(stream)))
        return C
