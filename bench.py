#!/usr/bin/env python3
"""Benchmark of one Kimi-K2 MLA layer on one MI355X, through the C ABI (libmla.so).

Headline workload (the largest configuration of the layer's workloads): FP8 weights (E4M3 codes,
one float32 scale per 128 x 128 block, dynamic 1 x 128 activation quantisation), decode of 128
sequences holding 16,384 cached positions each, one new token per sequence. A step is one decode
call: every stage of the decode path (activation quantisers, fused q_a|kv_a, both RMSNorms, RoPE
and the latent-cache append, q_b, the W_UK absorption, split attention over the 784-byte FP8
latent cache with its merge, W_UV, o_proj). `value` is µs per step.

`roofline` is the headline's dominant kernel, the split decode attention: algorithmic bytes per
launch (784 B per cached position, read once for all 64 heads) over its average duration,
measured in the same run with HIP events that the library records on the call's stream right
around that kernel (mla_test_probe_stage). `cpu_baseline` is the float64 oracle on a bounded
sample of the same workload.

Every other configuration is reported under "extra" with its own roofline record for its
dominant kernel(s) and its own CPU-oracle sample: prefill T=64 (C0), decode B=1 at position 1000
(C1), decode of 64 sequences with 1024..8192 cached positions (C2), prefill T=8192 (C3), FP8
prefill of 4 x 4096 (C4 prefill); also chunked prefill, YaRN decode, the decoder block's
attention half, the 61-layer cache pool and achievable peaks of this GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12       # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15      # flop/s, dense bf16 MFMA
FP8_PEAK = 5.0e15       # flop/s, dense fp8 MFMA

BF16_WEIGHT_BYTES = 2 * (1536 * 7168 + 1536 + 12288 * 1536 + 576 * 7168 + 512 + 16384 * 512 + 7168 * 8192)
OPROJ_BYTES = 2 * 7168 * 8192
PROJ_MACS_PER_TOKEN = 7168 * 2112 + 1536 * 12288 + 8192 * 7168  # q_a|kv_a, q_b, o_proj
KVB_MACS_PER_ROW = 512 * 16384


def attn_pairs(T, L0=0):
    """Causal (query, key) pairs of T new tokens after L0 cached positions."""
    return T * L0 + T * (T + 1) // 2


def prefill_flops(T, L0=0):
    """Algorithmic flops of a prefill of T tokens onto L0 cached positions: the projections of the
    T new tokens (kv_b on the T new latent rows), and 640 flop per head per causal pair (192-wide
    scores and 128-wide value mix). A cached prefix costs attention only."""
    proj = 2 * T * (PROJ_MACS_PER_TOKEN + KVB_MACS_PER_ROW)
    return proj + 640 * 64 * attn_pairs(T, L0)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Runner:
    def __init__(self, torch, binding):
        self.torch, self.binding = torch, binding

    def timed(self, fn, steps, warmup):
        """Wall time per call of `steps` calls after `warmup` untimed ones, bracketed by device syncs."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def probed(self, fn, steps, warmup, stage):
        """Average duration (s) of `stage` over `steps` calls: the library records a pair of HIP events
        on the call's stream right before and after that stage's launches (mla_test_probe_stage)."""
        torch, binding = self.torch, self.binding
        for i in range(warmup):
            fn(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:  # created on first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(steps):
            binding.probe_stage(stage, *evs[i])
            fn(warmup + i)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3


def roofline(kernel, bound, work, t, unit_work, note=""):
    """Roofline record: `work` algorithmic bytes (bound 'hbm') or flops (bound 'mfma-bf16'/'mfma-fp8')
    per launch over the launch's average duration t (s)."""
    if bound == "hbm":
        achieved, peak, unit = work / t / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = work / t / 1e12, (FP8_PEAK if bound == "mfma-fp8" else BF16_PEAK) / 1e12, "TFLOP/s"
    rec = {"kernel": kernel, "bound": "hbm" if bound == "hbm" else "mfma", "achieved": round(achieved, 1),
           "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "avg_launch_us": round(t * 1e6, 2),
           "work_per_launch": int(work), "work_unit": unit_work}
    if note:
        rec["note"] = note
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the headline's attention launches settle over the first ~40 steps of a fresh process (a kernel
    # trace shows 825 -> 585 us per launch: the GPU's clocks and power, not the work, change), so the
    # default warm-up puts the timed steps in the steady state the probed launches are measured in
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=3, help="bf16 layer copies stepped in turn")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="CPU work per oracle sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer is not sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from head_latent_attention_proj_amd import binding, synth

    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    R = Runner(torch, binding)
    extra = {}

    # ================= headline: FP8 decode, 128 sequences x 16384 cached positions
    log("FP8: generating weights and a 128 x 16384 cache")
    wq = synth.make_weights_fp8(seed=0)
    B8, P8 = 128, 16384
    n_calls = args.warmup + args.steps + 2 + args.steps  # timed loop, then the probed one
    lf = binding.Layer(binding.weights_to_device(wq), max_positions=P8 + n_calls + 1, wdtype=binding.WDTYPE_FP8)
    ents8 = torch.from_numpy(synth.make_cache_entries_fp8(P8, seed=2100)).cuda()
    c8 = binding.Cache(lf, [P8 + n_calls + 1] * B8)
    for s_ in range(B8):
        lf.cache_append(c8, s_, ents8)
    del ents8
    x8 = binding.bf16_tensor(synth.make_hidden(B8, seed=1005))
    y8 = torch.empty_like(x8)
    sid8h = np.arange(B8, dtype=np.int32)
    sid8d = torch.arange(B8, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def dec8(i):
        # each step appends one position per sequence (16385, 16386, ... positions attended)
        lf.decode(c8, sid8h, x8, y=y8, seq_ids_d=sid8d)

    log("timing FP8 decode B=128 x 16384")
    t_head = R.timed(dec8, args.steps, args.warmup)
    pos_head = P8 + args.warmup + (args.steps + 1) / 2  # mean positions attended per sequence, timed steps
    t_attn8 = R.probed(dec8, args.steps, 2, "decode_attn")
    pos_probe = P8 + args.warmup + args.steps + 2 + (args.steps + 1) / 2
    w8_bytes = sum(int(v.nbytes) for v in wq.values())
    head_bytes = w8_bytes + 784 * B8 * pos_head + 2 * 2 * 7168 * B8
    cache8 = 784 * B8 * pos_probe
    head_roof = roofline("decode_attn_fp8_kernel (FP8 latent cache, split attention)", "hbm", cache8, t_attn8,
                         f"bytes: 784 per cached position (all 64 heads), 128 x {pos_probe:.1f} positions on average")
    head_roof["traffic"] = counted_traffic("fp8_decode_attn")
    head_roof["step_share"] = round(t_attn8 / t_head, 3)
    del c8

    # ================= bf16 weight copies (own weights each; stepped in turn so the 202 MB of a
    # layer's weights cannot stay in the 256 MB Infinity Cache between its steps)
    log("generating bf16 weights")
    bits = synth.make_weights_bf16(seed=0)
    base = binding.weights_to_device(bits)
    layers = [binding.Layer(base if c == 0 else {k: v.clone() for k, v in base.items()}, max_positions=16384)
              for c in range(args.copies)]
    n_cp = len(layers)

    if not args.no_extra:
        # ---------------- C1: decode B=1 at position 1000 over 1000 cached positions (bf16)
        P0 = 1000
        steps1, warm1 = 60, 10
        caps = P0 + 400  # every call appends one position: C1 and block steps, plain and probed
        x_fill = binding.bf16_tensor(synth.make_hidden(P0, seed=1001))
        caches = []
        for L in layers:
            cache = binding.Cache(L, [caps])
            L.prefill(cache, [0], [0, P0], x_fill)
            caches.append(cache)
        x_new = binding.bf16_tensor(synth.make_hidden(1, seed=1002))
        y_new = torch.empty_like(x_new)
        sid_h = np.zeros(1, dtype=np.int32)
        sid_d = torch.zeros(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def dec1(i):
            c = i % n_cp
            layers[c].decode(caches[c], sid_h, x_new, y=y_new, seq_ids_d=sid_d)

        log("timing decode B=1")
        t1 = R.timed(dec1, steps1, warm1)
        # its o_proj kernel (M=1, N=7168, K=8192) on its own: a burst of back-to-back launches on the
        # layer copies' weights, bracketed by two HIP events on the stream (held by a sleep kernel until
        # the whole burst is queued, so neither host launch latency nor a probe event between kernels
        # is timed; a ~20 us kernel would see both)
        gemm = binding.Gemm()
        xo = binding.bf16_tensor(synth.make_activations(1, 8192, seed=7))
        yo = torch.empty((1, 7168), dtype=torch.bfloat16, device="cuda")
        for i in range(10):
            gemm(xo, layers[i % n_cp].weights["o"], yo, 1, 7168, 8192, stage="oproj")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        torch.cuda._sleep(20_000_000)
        e0.record(stream)
        for i in range(steps1):
            gemm(xo, layers[i % n_cp].weights["o"], yo, 1, 7168, 8192, stage="oproj")
        e1.record(stream)
        torch.cuda.synchronize()
        t1_op = e0.elapsed_time(e1) * 1e-3 / steps1
        b1 = BF16_WEIGHT_BYTES + 1152 * (P0 + 1) + 1152 + 2 * 2 * 7168
        op_bytes = OPROJ_BYTES + 2 * 8192 + 2 * 7168
        r1 = roofline("gemm_rows_kernel (o_proj, M=1, N=7168, K=8192, bf16)", "hbm", op_bytes, t1_op,
                      "bytes: o_proj weights + o + y; burst of launches bracketed by HIP events")
        r1["traffic"] = counted_traffic("oproj_decode_B1")
        extra["C1_decode_B1_pos1000"] = {
            "us_per_step": round(t1 * 1e6, 2), "step_bytes": int(b1), "step_hbm_frac": round(b1 / t1 / HBM_PEAK, 4),
            "roofline": r1,
            "note": "three layer copies stepped in turn (positions 1000, 1001, ... of each copy)"}

        # the same step as the attention half of a decoder block (input RMSNorm, residual in o_proj)
        log("timing block decode B=1")
        gain = binding.bf16_tensor(synth.make_block_norm(seed=7))
        h_new = torch.empty_like(x_new)

        def blk1(i):
            c = i % n_cp
            layers[c].block_decode(caches[c], sid_h, gain, x_new, h=h_new, seq_ids_d=sid_d)

        extra["block_decode_B1"] = {
            "us_per_step": round(R.timed(blk1, steps1, warm1) * 1e6, 2),
            "note": "decoder-block attention half h = x + MLA(RMSNorm(x)) on the C1 caches"}

        # YaRN RoPE (the released rope_scaling): the C1 step again
        log("timing YaRN decode B=1")
        ylayers = [binding.Layer(L.weights, max_positions=16384, rope_scaling=binding.KIMI_K2_YARN) for L in layers]
        ycaches = []
        for L in ylayers:
            cache = binding.Cache(L, [caps])
            L.prefill(cache, [0], [0, P0], x_fill)
            ycaches.append(cache)

        def ydec(i):
            c = i % n_cp
            ylayers[c].decode(ycaches[c], sid_h, x_new, y=y_new, seq_ids_d=sid_d)

        extra["yarn_decode_B1"] = {
            "us_per_step": round(R.timed(ydec, steps1, warm1) * 1e6, 2),
            "note": "C1 with YaRN RoPE (factor 32, original 4096, beta 1/1, mscale 1/1): only the rotary table and "
                    "the softmax scale differ"}
        del ylayers, ycaches, caches

        # ---------------- C0 and C3: prefill T=64 and T=8192 on an empty cache (bf16)
        for T, steps, warm, tag in ((64, 30, 5, "C0_prefill_T64"), (8192, 8, 3, "C3_prefill_T8192")):
            log(f"timing prefill T={T}")
            xb = binding.bf16_tensor(synth.make_hidden(T, seed=1003))
            pc = [binding.Cache(L, [T]) for L in layers]
            yb = torch.empty_like(xb)
            sid = np.zeros(1, dtype=np.int32)
            qs = np.array([0, T], dtype=np.int32)
            sid_dev = torch.from_numpy(sid).cuda()
            qs_dev = torch.from_numpy(qs).cuda()

            def pre(i, T=T, xb=xb, pc=pc, yb=yb, sid=sid, qs=qs, sid_dev=sid_dev, qs_dev=qs_dev):
                c = i % n_cp
                pc[c].len_h[0] = 0
                pc[c].len_d.zero_()
                layers[c].prefill(pc[c], sid, qs, xb, y=yb, seq_ids_d=sid_dev, q_start_d=qs_dev)

            t = R.timed(pre, steps, warm)
            fl = prefill_flops(T)
            rec = {"ms": round(t * 1e3, 4), "tokens_per_s": round(T / t, 1), "tflops": round(fl / t / 1e12, 2),
                   "mfma_frac": round(fl / t / BF16_PEAK, 4)}
            if T == 64:
                b0 = BF16_WEIGHT_BYTES + 1152 * T + 2 * 2 * 7168 * T
                rec.update({"step_bytes": int(b0), "step_hbm_frac": round(b0 / t / HBM_PEAK, 4)})
                rec["roofline"] = roofline("whole prefill step (weights dominate)", "hbm", b0, t,
                                           "bytes: weights + x + y + new entries")
            else:
                t_at = R.probed(pre, steps, 1, "prefill_attn")
                t_op = R.probed(pre, steps, 1, "oproj")
                rec["roofline"] = roofline("prefill_attn_kernel<false> (causal, bf16)", "mfma-bf16",
                                           640 * 64 * attn_pairs(T), t_at, "flops: 640 per head per causal pair")
                rec["roofline_oproj"] = roofline("gemm_tile_kernel (o_proj, M=8192, N=7168, K=8192, bf16)",
                                                 "mfma-bf16", 2 * T * 8192 * 7168, t_op, "flops: 2 M N K")
            rec["note"] = "includes one zero-fill of the device length per step"
            extra[tag] = rec
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

        def chunk(i):
            c = i % n_cp
            ccs[c].len_h[0] = L0c
            ccs[c].len_d.fill_(L0c)
            layers[c].prefill(ccs[c], sid, qs, xb, y=yb, seq_ids_d=sid_dev, q_start_d=qs_dev)

        t = R.timed(chunk, 20, 5)
        fl = prefill_flops(T, L0c)
        extra["prefill_chunk_T512_on_L3584"] = {
            "ms": round(t * 1e3, 4), "tokens_per_s": round(T / t, 1), "tflops": round(fl / t / 1e12, 2),
            "mfma_frac": round(fl / t / BF16_PEAK, 4),
            "note": "flops algorithmic: projections of the 512 new tokens and attention over 3,584 + causal keys; "
                    "the path also re-runs kv_b over the 3,584 cached rows, which is not counted"}
        del ccs, xb, yb, ent_c

        # ---------------- C2: decode B=64, lengths U[1024, 8192], a cache per layer copy
        log("timing decode B=64 varlen")
        B = 64
        lens = synth.make_lengths(B, 1024, 8192, seed=1002)
        ents = binding.bf16_tensor(synth.make_cache_entries(int(lens.max()), seed=2002))
        vcs = []
        for L in layers:
            vc = binding.Cache(L, lens + 8)
            for s in range(B):
                L.cache_append(vc, s, ents[: int(lens[s])])
            vcs.append(vc)
        del ents
        xb = binding.bf16_tensor(synth.make_hidden(B, seed=1004))
        yb = torch.empty_like(xb)
        sid_h64 = np.arange(B, dtype=np.int32)
        sid_d64 = torch.arange(B, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def dec64(i):
            c = i % n_cp
            layers[c].decode(vcs[c], sid_h64, xb, y=yb, seq_ids_d=sid_d64)
            vcs[c].len_h[:] = lens
            vcs[c].len_d.sub_(1)

        t = R.timed(dec64, 30, 20)  # the first steps of a burst run slower while clocks settle
        t_at = R.probed(dec64, 30, 2, "decode_attn")
        kv_bytes = 1152 * int(np.sum(lens + 1))
        byts = BF16_WEIGHT_BYTES + kv_bytes + 1152 * B + 2 * 2 * 7168 * B
        r2 = roofline("decode_attn_bf16_kernel (bf16 latent cache, split attention)", "hbm", kv_bytes, t_at,
                      "bytes: 1,152 per cached position (all 64 heads)")
        r2["traffic"] = counted_traffic("bf16_decode_attn")
        extra["C2_decode_B64_varlen"] = {
            "us_per_step": round(t * 1e6, 2), "step_bytes": int(byts), "step_hbm_frac": round(byts / t / HBM_PEAK, 4),
            "sum_len": int(lens.sum()), "roofline": r2,
            "note": "three layer copies with their own caches stepped in turn; lengths rewound after each step"}
        del vcs, xb, yb

        # ---------------- C4 prefill: FP8, 4 sequences x 4096 tokens
        log("timing FP8 prefill B=4 x T=4096")
        T8 = 4096
        xp8 = binding.bf16_tensor(synth.make_hidden(4 * T8, seed=1006))
        yp8 = torch.empty_like(xp8)
        cp8 = binding.Cache(lf, [T8] * 4)
        qs8 = np.arange(5, dtype=np.int32) * T8
        sids = np.arange(4, dtype=np.int32)
        sids_dev = torch.from_numpy(sids).cuda()
        qs8_dev = torch.from_numpy(qs8).cuda()

        def pre8(i):
            cp8.len_h[:] = 0
            cp8.len_d.zero_()
            lf.prefill(cp8, sids, qs8, xp8, y=yp8, seq_ids_d=sids_dev, q_start_d=qs8_dev)

        t = R.timed(pre8, 6, 2)
        t_at = R.probed(pre8, 3, 0, "prefill_attn")
        t_op = R.probed(pre8, 3, 0, "oproj")
        fl = 4 * prefill_flops(T8)
        proj_fp8 = 4 * 2 * T8 * (PROJ_MACS_PER_TOKEN + KVB_MACS_PER_ROW)
        att = 4 * 640 * 64 * attn_pairs(T8)
        extra["C4_prefill_B4_T4096_fp8"] = {
            "ms": round(t * 1e3, 3), "tokens_per_s": round(4 * T8 / t, 1), "tflops": round(fl / t / 1e12, 2),
            "mfma_frac": round((proj_fp8 / FP8_PEAK + att / BF16_PEAK) / t, 4),
            "roofline": roofline("prefill_attn_kernel<true> (causal, fp16 operands, value residuals)", "mfma-bf16", att,
                                 t_at, "flops: 640 per head per causal pair (counted once, though the value products "
                                       "run twice: values and their fp16 residuals)"),
            "roofline_oproj": roofline("gemm_fp8_ring_kernel (o_proj, M=16384, N=7168, K=8192, FP8 native)", "mfma-fp8",
                                       2 * 4 * T8 * 8192 * 7168, t_op, "flops: 2 M N K"),
            "note": "mfma_frac = (fp8 projection flops / 5 PF + attention flops / 2.5 PF) / time"}
        del cp8, xp8, yp8

        # ---------------- 61-layer cache pool: bytes per position (host-side layout plan)
        pool_bytes = {}
        for name, wd in (("bf16", binding.WDTYPE_BF16), ("fp8", binding.WDTYPE_FP8)):
            cfg = binding.make_config(wdtype=wd)
            cap1 = np.array([1], dtype=np.int32)
            off = np.zeros(1, dtype=np.int64)
            tot, lb, pb = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
            binding.check(binding.lib().mla_cache_pool_plan(ctypes.byref(cfg), 61, 1, cap1.ctypes.data, 1,
                                                             off.ctypes.data, ctypes.byref(tot), ctypes.byref(lb),
                                                             ctypes.byref(pb)))
            pool_bytes[name] = pb.value
        extra["cache_pool_61_layers"] = {
            "bytes_per_position_bf16": pool_bytes["bf16"], "bytes_per_position_fp8": pool_bytes["fp8"],
            "note": "mla_cache_pool_plan over 61 layers, one position; rebuilt keys and values would take 2,498,560 B"}

        # ---------------- achievable peaks of this GPU, for context next to the published ones
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
            "note": "context only; roofline fractions use the published 8 TB/s, 2.5 PF/s (bf16), 5 PF/s (fp8)"}

    # a plain 64 MiB device copy: the reference point that scales rocprofv3's FETCH_SIZE / WRITE_SIZE
    # counters to bytes (its algorithmic traffic is exactly 64 MiB read + 64 MiB written)
    cp_src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    del cp_src, cp_dst

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_fp8_decode(wq, args.cpu_seconds)
        if not args.no_extra:
            extra["cpu_oracle"] = {
                "C0_prefill_T64": cpu_prefill(bits, 64, args.cpu_seconds),
                "C1_decode_B1_pos1000": cpu_decode_b1(bits, args.cpu_seconds),
                "C2_decode_B64_varlen": cpu_decode_varlen(bits, args.cpu_seconds),
                "C3_prefill_T8192": cpu_prefill(bits, 8192, args.cpu_seconds),
                "C4_prefill_B4_T4096_fp8": cpu_prefill(wq, 4096, args.cpu_seconds, batch=4),
            }

    line = {
        "metric": "MLA layer prefill tokens/s + decode µs/step; % of HBM / MFMA roofline",
        "value": round(t_head * 1e6, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_head * 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded E4M3 weights with 128x128 scales 2^U(-10,-4), N(0,1) hidden states, random "
                "FP8 cache entries; random-init, no checkpoint)",
        "config": {
            "workload": "decode B=128, one new token per sequence over 16384 cached positions each, FP8 e4m3 "
                        "weights with 128x128 block scales and dynamic 1x128 activations, Kimi-K2 MLA layer "
                        "(hidden 7168, q_lora 1536, kv_lora 512, 64 heads, 128/64/128)",
            "global_batch": B8, "seq_len": round(pos_head, 1), "parallelism": "single GPU",
        },
        "step_bytes": int(head_bytes),
        "step_hbm_gbs": round(head_bytes / t_head / 1e9, 1),
        "step_hbm_frac": round(head_bytes / t_head / HBM_PEAK, 4),
        "roofline": head_roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


# ---- HBM traffic of the roofline kernels from committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes
# (profiles/*_traffic.json). A record stands only while the source text it names hashes to the
# recorded value (the kernel has not changed since the counters were taken); otherwise None.
def source_regions_sha256(path, regions):
    with open(os.path.join(ROOT, path)) as f:
        src = f.read()
    h = hashlib.sha256()
    for start, end in regions:
        i = src.index(start)
        h.update(src[i:src.index(end, i)].encode())
    return h.hexdigest()


def counted_traffic(name):
    try:
        with open(os.path.join(ROOT, "profiles", f"{name}_traffic.json")) as f:
            rec = json.load(f)
        sha = source_regions_sha256(rec["source"], rec["source_regions"])
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if sha == rec.get("source_regions_sha256") else None


# ---- CPU baselines: the float64 oracle as it stands, on bounded samples of each workload, timed on
# this host's cores (numpy BLAS threads), each scaled to its workload's unit and saying what ran.
def _blas_threads():
    from threadpoolctl import threadpool_info

    t = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
    return int(max(t)) if t else 1


def _w64(wbits):
    from head_latent_attention_proj_amd import synth
    from oracle import fp8 as ofp8

    if "q_a_s" in wbits:
        w = {n: ofp8.dequant_weight(wbits[n], wbits[n + "_s"]) for n in ("q_a", "q_b", "kv_a", "kv_b", "o")}
        for n in ("q_a_norm", "kv_a_norm"):
            w[n] = synth.bf16_bits_to_f64(wbits[n])
        return w, True
    return {k: synth.bf16_bits_to_f64(v) for k, v in wbits.items()}, False


def _rec(value, unit, sample):
    return {"value": round(float(value), 1), "unit": unit, "cores": _blas_threads(), "kind": "oracle", "sample": sample,
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_fp8_decode(wq, seconds):
    """C4 decode: the W8A8 oracle's decode step of single sequences at 16384 cached positions (rebuilt
    keys and values, the oracle's definition), as many as fit in `seconds`, times 128 sequences."""
    from head_latent_attention_proj_amd import synth
    from oracle import fp8 as ofp8
    from oracle import mla as omla

    w, _ = _w64(wq)
    raw = synth.make_cache_entries_fp8(16384, seed=2100)
    sc = np.ascontiguousarray(raw[:, 512:528]).view(np.float32)
    c = ofp8.dequant_1x128(raw[:, :512], sc)
    k = np.ascontiguousarray(raw[:, 528:]).view(np.float32).astype(np.float64)
    x = synth.bf16_bits_to_f64(synth.make_hidden(8, seed=1005))
    n, t0 = 0, time.perf_counter()
    while n < 8:
        omla.forward(x[n:n + 1], w, cache=(c, k), w8a8=True)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    return _rec(dt * 128 * 1e6, "us/step",
                f"{n} of the 128 sequences (float64 W8A8 decode over 16384 cached positions each), {dt * n:.1f} s, x128")


def cpu_decode_b1(bits, seconds):
    """C1: the oracle's decode step at position 1000 over 1000 cached entries, repeated for `seconds`."""
    from head_latent_attention_proj_amd import synth
    from oracle import mla as omla

    w, _ = _w64(bits)
    ents = synth.bf16_bits_to_f64(synth.make_cache_entries(1000, seed=2001))
    x = synth.bf16_bits_to_f64(synth.make_hidden(1, seed=1002))
    n, t0 = 0, time.perf_counter()
    while True:
        omla.forward(x, w, cache=(ents[:, :512], ents[:, 512:]))
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    return _rec(dt * 1e6, "us/step", f"{n} float64 decode steps at position 1000, {dt * n:.1f} s")


def cpu_decode_varlen(bits, seconds):
    """C2: single-sequence oracle decode steps at the workload's cached lengths (the first ones that fit
    in `seconds`); the step estimate scales their time by total / sampled cached positions."""
    from head_latent_attention_proj_amd import synth
    from oracle import mla as omla

    w, _ = _w64(bits)
    lens = synth.make_lengths(64, 1024, 8192, seed=1002)
    ents = synth.bf16_bits_to_f64(synth.make_cache_entries(int(lens.max()), seed=2002))
    x = synth.bf16_bits_to_f64(synth.make_hidden(64, seed=1004))
    n, t0 = 0, time.perf_counter()
    while n < 64:
        e = ents[: int(lens[n])]
        omla.forward(x[n:n + 1], w, cache=(e[:, :512], e[:, 512:]))
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    est = dt * float(np.sum(lens + 1)) / float(np.sum(lens[:n] + 1))
    return _rec(est * 1e6, "us/step", f"{n} of the 64 sequences ({int(np.sum(lens[:n]))} cached positions), "
                                      f"{dt:.1f} s, scaled by cached positions")


def cpu_prefill(wbits, T, seconds, batch=1):
    """Prefill of T tokens (per sequence; `batch` sequences): the oracle's latent path and rebuilt keys
    and values over all T tokens with the last row's output (one call, timed), then one call for n
    evenly spaced query rows up to the last (n doubled until that call takes half of `seconds`): the
    difference of the two calls is the attention of n - 1 more rows over T keys, and the estimate adds
    that cost per (row, key) pair times the T(T+1)/2 causal pairs of the sequence, times `batch`."""
    from head_latent_attention_proj_amd import synth
    from oracle import mla as omla

    w, fp8 = _w64(wbits)
    x = synth.bf16_bits_to_f64(synth.make_hidden(T, seed=1003))
    if T <= 64:
        n, t0 = 0, time.perf_counter()
        while True:
            omla.forward(x, w, w8a8=fp8)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / n
        return _rec(T / dt, "tokens/s", f"{n} float64 prefills of {T} tokens, {dt * n:.1f} s")
    t0 = time.perf_counter()
    omla.forward(x, w, rows=np.array([T - 1]), w8a8=fp8)
    t_base = time.perf_counter() - t0
    n = 8
    while True:
        rows = np.linspace(T // 8, T - 1, n).astype(int)
        t0 = time.perf_counter()
        omla.forward(x, w, rows=rows, w8a8=fp8)
        t_rows = time.perf_counter() - t0
        if t_rows - t_base >= seconds / 2 or n >= 512:
            break
        n *= 2
    per_pair = max(t_rows - t_base, 0.0) / ((n - 1) * T)
    est = batch * (t_base + per_pair * T * (T + 1) / 2)
    what = "W8A8 " if fp8 else ""
    return _rec(batch * T / est, "tokens/s",
                f"float64 {what}prefill of {T} tokens estimated from one call computing the kv path of all {T} "
                f"with one query row ({t_base:.1f} s) and one with {n} query rows over all {T} keys "
                f"({t_rows:.1f} s), x{batch} sequences")

if __name__ == "__main__":
    main()
