#!/usr/bin/env python3
"""Benchmark of one Kimi-K2 MLA layer on one MI355X, through the C ABI (libmla.so).

Headline workload: decode, batch 1, one new token at position 1000 over 1000 cached positions
(bf16 weights N(0, 0.02), gains 1 + N(0, 0.1), hidden states N(0, 1); the cache is filled by an
untimed GPU prefill of 1000 tokens). A step is one decode call, i.e. every stage of the decode
path: fused q_a|kv_a projection, both RMSNorms, RoPE and the latent-cache append, q_b, the W_UK
absorption, split attention over the latent cache with its merge, W_UV and o_proj.

Three copies of the layer (own weights, own cache) are stepped in turn, as consecutive layers of
a model are: the 202 MB of weights per layer then cannot sit in the 256 MB Infinity Cache
between its steps, so the step reads them from HBM.

Also reported (same process, same JSON line, under "extra"): prefill of 64 and 8192 tokens
(tokens/s, MFMA fraction) and batched decode of 64 sequences with cached lengths uniform in
[1024, 8192] (µs/step, HBM fraction). `roofline` is the o_proj kernel of the headline step timed
on its own with HIP events on its stream; `cpu_baseline` is the float64 oracle's decode step.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12       # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15      # flop/s, dense bf16 MFMA

WEIGHT_BYTES = 2 * (1536 * 7168 + 1536 + 12288 * 1536 + 576 * 7168 + 512 + 16384 * 512 + 7168 * 8192)
OPROJ_BYTES = 2 * 7168 * 8192


def decode_step_bytes(lens_after, B):
    """Algorithmic bytes of one decode step: weights once, 1,152 B per cached position read,
    the new entry written, x read and y written."""
    return WEIGHT_BYTES + 1152 * int(np.sum(lens_after)) + 1152 * B + 2 * 2 * 7168 * B


def prefill_flops(T):
    """Projections (2 * MACs) plus causal attention: 640 flop per head per causal pair."""
    proj = 2 * T * (7168 * 2112 + 1536 * 12288 + 512 * 16384 + 8192 * 7168)
    att = 640 * 64 * T * (T + 1) // 2
    return proj + att


def chunk_prefill_flops(T, L0):
    """Prefill of T tokens onto L0 cached positions as this path runs it: the projections of the T
    tokens, kv_b over all L0 + T latent rows (the cached prefix is up-projected again), and 640
    flop per head per causal pair (query t sees L0 + t + 1 keys)."""
    proj = 2 * T * (7168 * 2112 + 1536 * 12288 + 8192 * 7168) + 2 * (L0 + T) * 512 * 16384
    att = 640 * 64 * (T * L0 + T * (T + 1) // 2)
    return proj + att


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_loop(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3, help="layer copies stepped in turn")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer is not sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from head_latent_attention_proj_amd import binding, synth

    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    log("generating weights")
    bits = synth.make_weights_bf16(seed=0)
    base = binding.weights_to_device(bits)
    layers = []
    for c in range(args.copies):
        w = base if c == 0 else {k: v.clone() for k, v in base.items()}
        layers.append(binding.Layer(w, max_positions=16384))

    # ---------------- headline: decode B=1 at position 1000 over 1000 cached positions
    P0 = 1000
    total_steps = args.steps + args.warmup
    caps = P0 + 2 * (total_steps // args.copies + 2)  # the headline steps, then the block's
    caches, xs = [], []
    x_fill = binding.bf16_tensor(synth.make_hidden(P0, seed=1001))
    for c, L in enumerate(layers):
        cache = binding.Cache(L, [caps])
        L.prefill(cache, [0], [0, P0], x_fill)
        caches.append(cache)
    x_new = binding.bf16_tensor(synth.make_hidden(1, seed=1002))
    y_new = torch.empty_like(x_new)
    sid_h = np.zeros(1, dtype=np.int32)
    sid_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def decode_step(i):
        c = i % args.copies
        layers[c].decode(caches[c], sid_h, x_new, y=y_new, seq_ids_d=sid_d)

    log("timing decode B=1")
    t_dec = timed_loop(torch, decode_step, args.steps, args.warmup)
    us_per_step = t_dec * 1e6
    lens_after = np.array([P0 + 1])
    dec_bytes = decode_step_bytes(lens_after, 1)

    # ---------------- the same step as the attention half of a decoder block (input RMSNorm
    # before the layer, residual added in o_proj's epilogue), on the same caches
    log("timing block decode B=1")
    gain = binding.bf16_tensor(synth.make_block_norm(seed=7))
    h_new = torch.empty_like(x_new)

    def block_step(i):
        c = i % args.copies
        layers[c].block_decode(caches[c], sid_h, gain, x_new, h=h_new, seq_ids_d=sid_d)

    t_blk = timed_loop(torch, block_step, args.steps, args.warmup)

    # ---------------- roofline: o_proj kernel of that step, HIP events on its stream
    log("timing o_proj kernel")
    gemm = binding.Gemm()
    xo = binding.bf16_tensor(synth.make_activations(1, 8192, seed=7))
    yo = torch.empty((1, 7168), dtype=torch.bfloat16, device="cuda")
    n_ev = max(args.steps, 30)
    for i in range(10):
        gemm(xo, layers[i % args.copies].weights["o"], yo, 1, 7168, 8192, stage="oproj")
    # hold the stream for a few milliseconds so that the whole burst below is queued before its
    # first launch runs: the two events then bracket n_ev back-to-back kernels (weights rotated
    # over the layer copies), not the host's launch latency or per-launch event overhead
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record(stream)
    for i in range(n_ev):
        gemm(xo, layers[i % args.copies].weights["o"], yo, 1, 7168, 8192, stage="oproj")
    e1.record(stream)
    torch.cuda.synchronize()
    oproj_ms = e0.elapsed_time(e1) / n_ev
    oproj_bytes = OPROJ_BYTES + 2 * 8192 + 2 * 7168
    achieved = oproj_bytes / (oproj_ms * 1e-3) / 1e9
    traffic = counted_traffic()

    # latent cache of the whole 61-layer stack in one pool (host-side layout plan): bytes per position
    pool_bytes = {}
    for name, wd in (("bf16", binding.WDTYPE_BF16), ("fp8", binding.WDTYPE_FP8)):
        cfg = binding.make_config(wdtype=wd)
        caps = np.array([1], dtype=np.int32)
        off = np.zeros(1, dtype=np.int64)
        tot, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
        binding.check(binding.lib().mla_cache_pool_plan(ctypes.byref(cfg), 61, 1, caps.ctypes.data, 1,
                                                         off.ctypes.data, ctypes.byref(tot), ctypes.byref(lb),
                                                         ctypes.byref(pb)))
        pool_bytes[name] = pb.value
    extra = {"cache_pool_61_layers": {
        "bytes_per_position_bf16": pool_bytes["bf16"], "bytes_per_position_fp8": pool_bytes["fp8"],
        "note": "mla_cache_pool_plan over 61 layers, one position; the rebuilt keys and values would take 2,498,560 B"},
        "block_decode_B1": {
        "us_per_step": round(t_blk * 1e6, 3),
        "note": "decoder-block attention half h = x + MLA(RMSNorm(x)): input-norm kernel, the decode step, "
                "residual fused into o_proj; positions 1000+ on the headline caches"}}
    if not args.no_extra:
        # ---------------- prefill T=64 and T=8192
        for T, steps, warm in ((64, 30, 5), (8192, 10, 5)):
            log(f"timing prefill T={T}")
            xb = binding.bf16_tensor(synth.make_hidden(T, seed=1003))
            pc = [binding.Cache(L, [T]) for L in layers]
            yb = torch.empty_like(xb)
            sid = np.zeros(1, dtype=np.int32)
            qs = np.array([0, T], dtype=np.int32)
            sid_dev = torch.from_numpy(sid).cuda()
            qs_dev = torch.from_numpy(qs).cuda()

            def prefill_step(i, T=T, xb=xb, pc=pc, yb=yb, sid=sid, qs=qs, sid_dev=sid_dev, qs_dev=qs_dev):
                c = i % args.copies
                pc[c].len_h[0] = 0
                pc[c].len_d.zero_()
                layers[c].prefill(pc[c], sid, qs, xb, y=yb, seq_ids_d=sid_dev, q_start_d=qs_dev)

            t = timed_loop(torch, prefill_step, steps, warm)
            fl = prefill_flops(T)
            extra[f"prefill_T{T}"] = {
                "ms": round(t * 1e3, 4), "tokens_per_s": round(T / t, 1),
                "tflops": round(fl / t / 1e12, 2), "mfma_frac": round(fl / t / BF16_PEAK, 4),
                "note": "includes one zero-fill of the device length per step",
            }
            del pc, xb, yb
        # ---------------- chunked prefill: 512 new tokens onto 3,584 cached positions
        log("timing chunked prefill T=512 onto 3584 cached positions")
        T, L0c = 512, 3584
        ent_c = binding.bf16_tensor(synth.make_cache_entries(L0c, seed=2003))
        ccs = []
        for L in layers:
            cc = binding.Cache(L, [L0c + T])
            L.cache_append(cc, 0, ent_c)
            ccs.append(cc)
        xb = binding.bf16_tensor(synth.make_hidden(T, seed=1005))
        yb = torch.empty_like(xb)
        sid = np.zeros(1, dtype=np.int32)
        qs = np.array([0, T], dtype=np.int32)
        sid_dev = torch.from_numpy(sid).cuda()
        qs_dev = torch.from_numpy(qs).cuda()

        def chunk_step(i):
            c = i % args.copies
            ccs[c].len_h[0] = L0c
            ccs[c].len_d.fill_(L0c)
            layers[c].prefill(ccs[c], sid, qs, xb, y=yb, seq_ids_d=sid_dev, q_start_d=qs_dev)

        t = timed_loop(torch, chunk_step, 20, 5)
        fl = chunk_prefill_flops(T, L0c)
        extra["prefill_chunk_T512_on_L3584"] = {
            "ms": round(t * 1e3, 4), "tokens_per_s": round(T / t, 1),
            "tflops": round(fl / t / 1e12, 2), "mfma_frac": round(fl / t / BF16_PEAK, 4),
            "note": "512 new tokens of one sequence after 3,584 cached positions (synthetic entries); kv_b "
                    "rebuilds keys and values for all 4,096 rows; includes one fill of the device length per step"}
        del ccs, xb, yb, ent_c
        # ---------------- YaRN RoPE (the released rope_scaling): the decode B=1 step again
        log("timing YaRN decode B=1")
        ylayers = [binding.Layer(L.weights, max_positions=16384, rope_scaling=binding.KIMI_K2_YARN) for L in layers]
        ycaches = []
        for L in ylayers:
            cache = binding.Cache(L, [P0 + args.steps + args.warmup + 2])
            L.prefill(cache, [0], [0, P0], x_fill)
            ycaches.append(cache)

        def yarn_step(i):
            c = i % args.copies
            ylayers[c].decode(ycaches[c], sid_h, x_new, y=y_new, seq_ids_d=sid_d)

        t = timed_loop(torch, yarn_step, args.steps, args.warmup)
        extra["yarn_decode_B1"] = {
            "us_per_step": round(t * 1e6, 3),
            "note": "decode B=1 at position 1000 with YaRN RoPE (factor 32, original 4096, beta 1/1, mscale 1/1): "
                    "only the rotary table and the softmax scale differ, so the kernels are the headline's"}
        del ylayers, ycaches
        # ---------------- decode B=64, lengths U[1024, 8192]
        log("timing decode B=64 varlen")
        B = 64
        lens = synth.make_lengths(B, 1024, 8192, seed=1002)
        L0 = layers[0]
        vc = binding.Cache(L0, lens + 8)
        ents = synth.make_cache_entries(int(lens.max()), seed=2002)
        ent_t = binding.bf16_tensor(ents)
        for s in range(B):
            L0.cache_append(vc, s, ent_t[: int(lens[s])])
        xb = binding.bf16_tensor(synth.make_hidden(B, seed=1004))
        yb = torch.empty_like(xb)
        sid_h64 = np.arange(B, dtype=np.int32)
        sid_d64 = torch.arange(B, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def dec64(i):
            # every step sees the same state: rewind the lengths by one after each step
            L0.decode(vc, sid_h64, xb, y=yb, seq_ids_d=sid_d64)
            vc.len_h[:] = lens
            vc.len_d.sub_(1)

        t = timed_loop(torch, dec64, 30, 20)  # 20 untimed steps: clocks settle (the first steps run slower)
        byts = decode_step_bytes(lens + 1, B)
        extra["decode_B64_varlen"] = {
            "us_per_step": round(t * 1e6, 2), "bytes": int(byts),
            "hbm_gbs": round(byts / t / 1e9, 1), "hbm_frac": round(byts / t / HBM_PEAK, 4),
            "sum_len": int(lens.sum()),
            "note": "one copy of the weights (MALL may hold part of them); includes one length rewind per step",
        }

    if not args.no_extra and not args.no_fp8:
        # ---------------- FP8 weights (E4M3, 128x128 block scales): decode B=128 x 16384 cached
        # positions, prefill B=4 x T=4096
        log("FP8: generating weights and a 128 x 16384 cache")
        wq = synth.make_weights_fp8(seed=0)
        lf = binding.Layer(binding.weights_to_device(wq), max_positions=16448, wdtype=binding.WDTYPE_FP8)
        B8, P8 = 128, 16384
        ents8 = torch.from_numpy(synth.make_cache_entries_fp8(P8, seed=2100)).cuda()
        c8 = binding.Cache(lf, [P8 + 1] * B8)
        for s_ in range(B8):
            lf.cache_append(c8, s_, ents8)
        del ents8
        x8 = binding.bf16_tensor(synth.make_hidden(B8, seed=1005))
        y8 = torch.empty_like(x8)
        sid8h = np.arange(B8, dtype=np.int32)
        sid8d = torch.arange(B8, dtype=torch.int32, device="cuda")
        lens8 = np.full(B8, P8, dtype=np.int32)
        torch.cuda.synchronize()

        def dec8(i):
            lf.decode(c8, sid8h, x8, y=y8, seq_ids_d=sid8d)
            c8.len_h[:] = lens8
            c8.len_d.sub_(1)

        log("timing FP8 decode B=128 x 16384")
        t = timed_loop(torch, dec8, 12, 8)
        w8_bytes = sum(int(v.nbytes) for k, v in wq.items())
        byts = w8_bytes + 784 * B8 * (P8 + 1) + 2 * 2 * 7168 * B8
        extra["fp8_decode_B128_L16384"] = {
            "us_per_step": round(t * 1e6, 2), "bytes": int(byts),
            "hbm_gbs": round(byts / t / 1e9, 1), "hbm_frac": round(byts / t / HBM_PEAK, 4),
            "note": "784-byte FP8 cache slots (synthetic codes); includes one length rewind per step",
        }
        del c8
        log("timing FP8 prefill B=4 x T=4096")
        T8 = 4096
        xp8 = binding.bf16_tensor(synth.make_hidden(4 * T8, seed=1006))
        yp8 = torch.empty_like(xp8)
        cp8 = binding.Cache(lf, [T8] * 4)
        qs8 = np.arange(5, dtype=np.int32) * T8
        sids = np.arange(4, dtype=np.int32)

        sids_dev = torch.from_numpy(np.ascontiguousarray(sids, dtype=np.int32)).cuda()
        qs8_dev = torch.from_numpy(np.ascontiguousarray(qs8, dtype=np.int32)).cuda()

        def pre8(i):
            cp8.len_h[:] = 0
            cp8.len_d.zero_()
            lf.prefill(cp8, sids, qs8, xp8, y=yp8, seq_ids_d=sids_dev, q_start_d=qs8_dev)

        t = timed_loop(torch, pre8, 3, 1)
        fl = 4 * prefill_flops(T8)
        extra["fp8_prefill_B4_T4096"] = {
            "ms": round(t * 1e3, 3), "tokens_per_s": round(4 * T8 / t, 1), "tflops": round(fl / t / 1e12, 2),
            "note": "flops count projections and causal attention once; o_proj runs on FP8 MFMA, the "
                    "other projections on bf16 MFMA over exactly widened codes, attention at split precision",
        }
        del cp8, lf

    # achievable peaks on this GPU, for context next to the published ones: a plain 1 GiB device copy
    # (bytes read + written per second) and a library bf16 GEMM (hipBLASLt through torch.matmul, 8192^3)
    if not args.no_extra:
        log("timing achievable peaks")
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        a_ = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        b_ = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a_, b_)
        e0.record()
        for _ in range(10):
            torch.matmul(a_, b_)
        e1.record()
        torch.cuda.synchronize()
        mm_tfs = 2 * 8192 ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del a_, b_
        extra["achievable_peaks"] = {
            "device_copy_GBps": round(copy_gbs, 1), "hipblaslt_bf16_gemm_8192_TFps": round(mm_tfs, 1),
            "note": "measured here for context; roofline fractions use the published 8 TB/s and 2.5 PF/s"}

    # a plain 64 MiB device copy: the reference point that scales rocprofv3's FETCH_SIZE / WRITE_SIZE
    # counters to bytes (its algorithmic traffic is exactly 64 MiB read + 64 MiB written)
    cp_src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    del cp_src, cp_dst

    cpu = None
    if not args.no_cpu:
        log("timing CPU oracle decode step")
        cpu = cpu_baseline(bits, args.cpu_seconds)

    line = {
        "metric": "MLA layer prefill tokens/s + decode µs/step; % of HBM / MFMA roofline",
        "value": round(us_per_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_dec * 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden states; random-init, no checkpoint)",
        "config": {
            "workload": "decode B=1, one new token at position 1000 over 1000 cached positions, "
                        "Kimi-K2 MLA layer (hidden 7168, q_lora 1536, kv_lora 512, 64 heads, 128/64/128), bf16",
            "global_batch": 1, "seq_len": P0 + 1, "parallelism": "single GPU", "layer_copies": args.copies,
        },
        "step_bytes": int(dec_bytes),
        "step_hbm_gbs": round(dec_bytes / t_dec / 1e9, 1),
        "step_hbm_frac": round(dec_bytes / t_dec / HBM_PEAK, 4),
        "roofline": {
            "kernel": "o_proj GEMM (M=1, N=7168, K=8192, bf16 weights)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
            "frac": round(achieved / 8000.0, 4), "traffic": traffic,
            "avg_launch_us": round(oproj_ms * 1e3, 3), "bytes_per_launch": int(oproj_bytes),
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


# Source text the roofline kernel's launches depend on: the epilogue, the row-streaming kernel's
# section and the launch planner of gemm.hip. The committed counter readings stand only while
# this text is unchanged.
ROOFLINE_SOURCE = "head_latent_attention_proj_amd/csrc/gemm.hip"
ROOFLINE_REGIONS = (("MLA_DEV void epi_store(", "\n}\n"),
                    ("// M <= 2: whole weight-row segments per load", "// Per-head products"),
                    ("Plan plan_gemm(", "\n}\n"))


def roofline_source_sha256():
    import hashlib

    with open(os.path.join(ROOT, ROOFLINE_SOURCE)) as f:
        src = f.read()
    h = hashlib.sha256()
    for start, end in ROOFLINE_REGIONS:
        i = src.index(start)
        h.update(src[i:src.index(end, i)].encode())
    return h.hexdigest()


def counted_traffic():
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    passes (profiles/oproj_decode_B1_bf16_pmc.md), or None when the kernel's source has changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", "oproj_decode_B1_bf16_traffic.json")) as f:
            rec = json.load(f)
        sha = roofline_source_sha256()
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if sha == rec.get("source_regions_sha256") else None


def cpu_baseline(bits, seconds):
    """The float64 oracle's decode step (position 1000, 1000 cached entries) on the host cores."""
    from threadpoolctl import threadpool_info

    from head_latent_attention_proj_amd import synth
    from oracle import mla as omla

    w64 = {k: synth.bf16_bits_to_f64(v) for k, v in bits.items()}
    ents = synth.bf16_bits_to_f64(synth.make_cache_entries(1000, seed=2001))
    x = synth.bf16_bits_to_f64(synth.make_hidden(1, seed=1002))
    cache = (ents[:, :512], ents[:, 512:])
    n, t0 = 0, time.perf_counter()
    while True:
        omla.forward(x, w64, cache=cache)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    threads = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {
        "value": round(dt * 1e6, 1), "unit": "us/step", "cores": int(max(threads) if threads else 1),
        "kind": "oracle",
        "sample": f"{n} float64 decode steps (position 1000 over 1000 cached entries), {dt * n:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
    }


if __name__ == "__main__":
    main()
