"""Pins of the float64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test ties one part of the oracle to something other than itself: numbers printed on the
pages (tests/golden/page_facts.json), closed forms, invariants, library routines and a
pure-Python brute force.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, fp8, mla

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))

TINY = mla.Config(hidden=8, q_lora=6, kv_lora=4, heads=2, nope=3, rope=4, v=2, eps=1e-6, theta=50000.0)


def tiny_weights(cfg: mla.Config, seed=3, zero=()):
    rng = np.random.default_rng(seed)
    w = {}
    for name, shape in mla.weight_shapes(cfg).items():
        if name.endswith("norm"):
            w[name] = 1.0 + 0.1 * rng.standard_normal(shape)
        else:
            w[name] = 0.5 * rng.standard_normal(shape)
        if name in zero:
            w[name] = np.zeros(shape)
    return w


def to_lists(w):
    return {k: v.tolist() for k, v in w.items()}


# ------------------------------------------------------------------------------------ P1, P2, P3
def test_parameter_counts_match_pages():
    g = GOLD["param_counts"]
    n = {k: int(np.prod(s)) for k, s in mla.weight_shapes().items()}
    cfg = mla.KIMI_K2
    kva_latent_rows = cfg.kv_lora * cfg.hidden
    kva_rope_rows = cfg.rope * cfg.hidden
    w_uk = cfg.heads * cfg.nope * cfg.kv_lora
    w_uv = cfg.heads * cfg.v * cfg.kv_lora
    assert n["q_a"] + n["q_a_norm"] == g["query_compression"]
    assert kva_latent_rows + n["kv_a_norm"] == g["kv_compression"]
    assert n["q_b"] == g["query_heads"]
    assert w_uk + kva_rope_rows == g["key_heads"]
    assert w_uv == g["value_heads"]
    assert n["o"] == g["causal_attention_out"]
    assert sum(n.values()) == g["per_instance_total"]
    assert n["kv_b"] == w_uk + w_uv
    assert w_uk == g["w_uk"] and 60 * w_uk == g["w_uk_times_60_moe_blocks"]


def test_cache_bytes_match_pages():
    g = GOLD["cache_bytes_per_token_61_layers"]
    b = mla.cache_bytes_per_position()
    assert b["rebuilt"] * g["layers"] == g["rebuilt_bf16"]
    assert b["latent"] * g["layers"] == g["latent_bf16"]
    assert b["flash_padded"] * g["layers"] == g["flash_padded_bf16"]
    assert round(b["rebuilt"] / b["latent"]) == g["ratio_rounded"]
    vp = GOLD["values_per_position"]
    assert b["rebuilt"] // 2 == vp["rebuilt"] and b["latent"] // 2 == vp["latent"]


def test_decode_shapes_at_position_1000():
    """1000 cached + 1 new token: rebuilt keys/values cover 1,001 positions ('KV cache' page)."""
    cfg = mla.KIMI_K2
    rng = np.random.default_rng(0)
    c_hat = rng.standard_normal((1001, cfg.kv_lora))
    k_pe = rng.standard_normal((1001, cfg.rope))
    w_kvb = 0.02 * rng.standard_normal(mla.weight_shapes()["kv_b"])
    k, v = mla.rebuild_kv(c_hat, k_pe, w_kvb)
    gk, gv = GOLD["decode_shapes_at_p1000"]["k"], GOLD["decode_shapes_at_p1000"]["v"]
    # the pages' layout is [B, heads, positions, features]; the oracle keeps [positions, heads, features]
    assert (k.shape[1], k.shape[0], k.shape[2]) == tuple(gk[1:])
    assert (v.shape[1], v.shape[0], v.shape[2]) == tuple(gv[1:])
    assert cfg.kv_lora == GOLD["tensor_shapes"]["latent"]
    assert cfg.heads * cfg.nope == GOLD["tensor_shapes"]["k_content_flat"]
    assert cfg.rope // 2 == GOLD["tensor_shapes"]["rope_pairs"]
    # the shared rotary key is the same in every head
    assert np.array_equal(k[:, 0, cfg.nope:], k[:, 63, cfg.nope:])


def test_kv_b_head_split_is_content_then_value():
    """W_UK is output features 0..127 of each head's 256 ('Key content up-projection', Explanation)."""
    cfg = mla.KIMI_K2
    rng = np.random.default_rng(1)
    c = rng.standard_normal((2, cfg.kv_lora))
    w_kvb = rng.standard_normal(mla.weight_shapes()["kv_b"])
    k, v = mla.rebuild_kv(c, np.zeros((2, cfg.rope)), w_kvb)
    h = 37
    assert np.allclose(k[:, h, :cfg.nope], c @ w_kvb[h * 256: h * 256 + 128].T, rtol=0, atol=1e-10)
    assert np.allclose(v[:, h], c @ w_kvb[h * 256 + 128: h * 256 + 256].T, rtol=0, atol=1e-10)


# ------------------------------------------------------------------------------------ P4 RMSNorm
def test_rmsnorm_identities():
    rng = np.random.default_rng(2)
    m, eps = 512, 1e-6
    x = rng.standard_normal((5, m))
    ones = np.ones(m)
    y = mla.rmsnorm(x, ones, eps)
    ms_x = np.mean(x * x, axis=1)
    # with unit gain, mean(y^2) = ms / (ms + eps)
    assert np.allclose(np.mean(y * y, axis=1), ms_x / (ms_x + eps), rtol=1e-13, atol=0)
    # odd symmetry, and scale invariance as eps -> 0
    assert np.array_equal(mla.rmsnorm(-x, ones, eps), -y)
    assert np.allclose(mla.rmsnorm(1000 * x, ones, 0.0), mla.rmsnorm(x, ones, 0.0), rtol=1e-13)
    # constant vector a*1 maps to g * a / sqrt(a^2 + eps)
    a = 0.003
    g = 1.0 + 0.1 * rng.standard_normal(m)
    assert np.allclose(mla.rmsnorm(np.full(m, a), g, eps), g * a / math.sqrt(a * a + eps), rtol=1e-14)
    # eps inside the root: for a tiny input the output is x / sqrt(eps), not x / (rms + eps)
    t = np.full(m, 1e-9)
    assert np.allclose(mla.rmsnorm(t, ones, eps), t / math.sqrt(1e-18 + eps), rtol=1e-12)


# ------------------------------------------------------------------------------------ P7 RoPE
def test_rope_matches_complex_rotation():
    cfg = mla.KIMI_K2
    rng = np.random.default_rng(4)
    pos = np.array([0, 1, 7, 1000, 131071])
    v = rng.standard_normal((len(pos), 3, cfg.rope))
    cos, sin = mla.rope_cos_sin(pos, cfg.rope, cfg.theta)
    r = mla.rope_rotate(v, cos, sin)
    z = v[..., 0::2] + 1j * v[..., 1::2]
    freq = np.array([cfg.theta ** (-(2 * i) / cfg.rope) for i in range(cfg.rope // 2)])
    rot = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    assert np.allclose(r[..., 0::2], rot.real, atol=1e-12) and np.allclose(r[..., 1::2], rot.imag, atol=1e-12)
    # position 0 is the identity; pair 0 turns by exactly p radians; pair 16 by p / sqrt(50000)
    assert np.array_equal(r[0], v[0])
    assert np.isclose(cos[3, 0], math.cos(1000.0)) and np.isclose(sin[3, 16], math.sin(1000.0 / math.sqrt(50000.0)))


def test_rope_relative_position_invariance():
    cfg = mla.KIMI_K2
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, cfg.rope))
    k = rng.standard_normal((1, cfg.rope))
    def score(pq, pk):
        cq, sq = mla.rope_cos_sin(np.array([pq]), cfg.rope, cfg.theta)
        ck, sk = mla.rope_cos_sin(np.array([pk]), cfg.rope, cfg.theta)
        return float((mla.rope_rotate(q, cq, sq) @ mla.rope_rotate(k, ck, sk).T)[0, 0])
    base = score(17, 5)
    for delta in (1, 100, 10000):
        assert abs(score(17 + delta, 5 + delta) - base) < 1e-9 * (1 + abs(base))
    # norms of pairs are preserved
    c, s = mla.rope_cos_sin(np.array([12345]), cfg.rope, cfg.theta)
    r = mla.rope_rotate(q, c, s)
    assert np.allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, q[:, 0::2] ** 2 + q[:, 1::2] ** 2, rtol=1e-13)


# ------------------------------------------------------------------------------------ YaRN RoPE
# The config excerpt ("KV cache" page) sets rope_scaling to YaRN: factor 32, original 4,096
# positions, beta_fast = beta_slow = 1, mscale = mscale_all_dim = 1. The pages give only these
# parameters; the rule itself is the YaRN paper's (Peng et al. 2023): per-pair interpolation by
# turns over the original context ("NTK-by-parts") and the attention factor 0.1 m ln(s) + 1.
def _plain_freq(cfg):
    return cfg.theta ** (-2.0 * np.arange(cfg.rope // 2) / cfg.rope)


def test_yarn_factor_one_is_plain_rope():
    pos = np.array([0, 3, 4095, 4096, 70000])
    plain = mla.rope_cos_sin(pos, 64, 50000.0)
    for cfg in (mla.Config(rope_factor=1.0), mla.Config(rope_factor=0.5)):
        c, s_ = mla.rope_cos_sin(pos, 64, 50000.0, cfg)
        assert np.array_equal(c, plain[0]) and np.array_equal(s_, plain[1])
        assert cfg.sigma == mla.KIMI_K2.sigma and cfg.rope_gain == 1.0


def test_yarn_released_config_is_a_step_at_one_turn():
    cfg = mla.KIMI_K2_YARN
    f = mla.yarn_frequencies(cfg.rope, cfg.theta, cfg.rope_factor, cfg.rope_orig_max, cfg.beta_fast, cfg.beta_slow)
    # a pair completes one turn over 4,096 positions when theta^(-2i/64) = 2 pi / 4096, i.e. at
    # i = 32 ln(4096 / 2 pi) / ln(50000) = 19.16: pairs 0..19 turn more often and keep their
    # frequency, pairs 20..31 are slowed by the factor 32
    i_turn = 32 * math.log(4096 / (2 * math.pi)) / math.log(50000.0)
    assert 19 < i_turn < 20
    ratio = f / _plain_freq(cfg)
    assert np.array_equal(ratio[:20], np.ones(20))
    assert np.allclose(ratio[20:], 1 / 32, rtol=1e-15)


def test_yarn_interpolated_pairs_replay_plain_rope_at_scaled_positions():
    # an interpolated pair at position 32 p has the plain angle of position p; an extrapolated
    # pair has the plain angle at the same position
    cfg = mla.KIMI_K2_YARN
    p = np.array([1, 100, 4095])
    cy, sy = mla.rope_cos_sin(32 * p, cfg.rope, cfg.theta, cfg)
    cp, sp = mla.rope_cos_sin(p, cfg.rope, cfg.theta)
    assert np.allclose(cy[:, 20:], cp[:, 20:], atol=1e-12) and np.allclose(sy[:, 20:], sp[:, 20:], atol=1e-12)
    cy1, _ = mla.rope_cos_sin(p, cfg.rope, cfg.theta, cfg)
    assert np.array_equal(cy1[:, :20], cp[:, :20])


def test_yarn_ramp_between_thresholds():
    # the paper's LLaMA thresholds (1 and 32 turns): frequencies fall monotonically from the
    # plain ones (pairs turning >= 32 times) to plain / s (pairs turning <= once)
    cfg = mla.Config(rope_factor=16.0, beta_fast=32.0, beta_slow=1.0)
    f = mla.yarn_frequencies(cfg.rope, cfg.theta, cfg.rope_factor, cfg.rope_orig_max, cfg.beta_fast, cfg.beta_slow)
    base = _plain_freq(cfg)
    turns = cfg.rope_orig_max * base / (2 * math.pi)
    ratio = f / base
    assert np.all(np.diff(ratio) <= 1e-15)
    assert np.array_equal(ratio[turns >= 32], np.ones(int((turns >= 32).sum())))
    assert np.allclose(ratio[turns <= 1], 1 / 16, rtol=1e-15)
    mid = (turns > 1) & (turns < 32)
    assert mid.sum() >= 3 and np.all((ratio[mid] > 1 / 16) & (ratio[mid] < 1))
    # at r = (1 + 32) / 2 the blend would be exactly halfway: check the pair closest to it lies
    # on the right side of the midpoint value
    j = int(np.argmin(np.abs(turns - 16.5)))
    half = (1 + 1 / 16) / 2
    assert (ratio[j] - half) * (turns[j] - 16.5) >= 0


def test_yarn_attention_factor_and_scale():
    cfg = mla.KIMI_K2_YARN
    f = 1 + 0.5 * math.log(2)  # 0.1 * ln 32 + 1, ln 32 = 5 ln 2
    assert mla.yarn_attention_factor(32.0, 1.0) == pytest.approx(f, rel=1e-15)
    assert cfg.sigma == pytest.approx(f * f / math.sqrt(192), rel=1e-15)
    assert cfg.rope_gain == 1.0
    assert mla.yarn_attention_factor(1.0, 1.0) == 1.0
    g = mla.Config(rope_factor=32.0, mscale=2.0, mscale_all_dim=1.0)
    assert g.rope_gain == pytest.approx((1 + math.log(2)) / f, rel=1e-15)
    assert mla.Config(rope_factor=32.0, scale=0.125).sigma == 0.125


def test_yarn_scores_depend_on_relative_position():
    cfg = mla.KIMI_K2_YARN
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, cfg.rope))
    k = rng.standard_normal((1, cfg.rope))
    def score(pq, pk):
        cq, sq = mla.rope_cos_sin(np.array([pq]), cfg.rope, cfg.theta, cfg)
        ck, sk = mla.rope_cos_sin(np.array([pk]), cfg.rope, cfg.theta, cfg)
        return float((mla.rope_rotate(q, cq, sq) @ mla.rope_rotate(k, ck, sk).T)[0, 0])
    base = score(5000, 4990)
    for delta in (1, 1000, 100000):
        assert abs(score(5000 + delta, 4990 + delta) - base) < 1e-9 * (1 + abs(base))


# ------------------------------------------------------------------------------------ P6 brute force
@pytest.mark.parametrize("t_new,l0", [(1, 0), (5, 0), (1, 4), (3, 2)])
def test_brute_force_tiny(t_new, l0):
    cfg = TINY
    w = tiny_weights(cfg)
    rng = np.random.default_rng(10 + t_new + 7 * l0)
    x_prev = rng.standard_normal((l0, cfg.hidden))
    x = rng.standard_normal((t_new, cfg.hidden))
    cache = mla.kv_entries(x_prev, w, 0, cfg) if l0 else None
    out = mla.forward(x, w, cfg, cache=cache)
    dims = dict(q_lora=cfg.q_lora, kv_lora=cfg.kv_lora, heads=cfg.heads, nope=cfg.nope, rope=cfg.rope, v=cfg.v)
    bcache = None
    if l0:
        bcache = [(list(cache[0][i]), list(cache[1][i])) for i in range(l0)]
    ys, ents = brute.forward(x.tolist(), to_lists(w), dims, cfg.eps, cfg.theta, 1 / math.sqrt(cfg.qk), bcache)
    assert np.allclose(out["y"], np.array(ys), rtol=0, atol=1e-12)
    assert np.allclose(out["c_hat"], np.array([e[0] for e in ents]), rtol=0, atol=1e-12)
    assert np.allclose(out["k_pe"], np.array([e[1] for e in ents]), rtol=0, atol=1e-12)


def test_brute_force_tiny_softmax_scale_default():
    assert mla.KIMI_K2.sigma == pytest.approx(1 / math.sqrt(192), rel=1e-15)


# ------------------------------------------------------------------------------------ P5 T = 1
def test_single_token_closed_form():
    """One token, empty cache: softmax over one key is 1, so o = W_UV,h c_hat for each head."""
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=11)
    x = np.random.default_rng(12).standard_normal((1, cfg.hidden))
    out = mla.forward(x, w, cfg)
    ckv = x[0] @ w["kv_a"].T
    c = ckv[: cfg.kv_lora]
    c_hat = w["kv_a_norm"] * c / math.sqrt(np.mean(c ** 2) + cfg.eps)
    kv = w["kv_b"] @ c_hat
    o = np.concatenate([kv[h * (cfg.nope + cfg.v) + cfg.nope:(h + 1) * (cfg.nope + cfg.v)] for h in range(cfg.heads)])
    assert np.allclose(out["y"][0], w["o"] @ o, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ P12 uniform
def test_uniform_attention_when_queries_vanish():
    """Zero q_b: every score is 0, so each query averages the values of positions 0..t."""
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=13, zero=("q_b",))
    x = np.random.default_rng(14).standard_normal((6, cfg.hidden))
    out = mla.forward(x, w, cfg)
    _, v = mla.rebuild_kv(out["c_hat"], out["k_pe"], w["kv_b"], cfg)
    for t in range(6):
        o = v[: t + 1].mean(axis=0).reshape(-1)
        assert np.allclose(out["y"][t], w["o"] @ o, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ P8 absorption
def test_absorbed_form_equals_rebuilt_form():
    cfg = mla.Config(hidden=96, q_lora=48, kv_lora=32, heads=4, nope=16, rope=8, v=12)
    w = tiny_weights(cfg, seed=15)
    x = np.random.default_rng(16).standard_normal((7, cfg.hidden))
    out = mla.forward(x, w, cfg)
    pos = np.arange(7)
    o_abs = mla.attend_absorbed(out["q_nope"], out["q_pe"], out["c_hat"], out["k_pe"], w["kv_b"], pos, cfg)
    assert np.allclose(o_abs.reshape(7, -1), out["o"], rtol=0, atol=1e-12)


def test_forward_absorbed_option_equals_rebuilt_forward():
    """forward(absorbed=True) (latent-space attention) against the rebuilt form, with a cached
    prefix and a subset of query rows."""
    cfg = mla.Config(hidden=96, q_lora=48, kv_lora=32, heads=4, nope=16, rope=8, v=12)
    w = tiny_weights(cfg, seed=61)
    rng = np.random.default_rng(62)
    x0 = rng.standard_normal((5, cfg.hidden))
    x1 = rng.standard_normal((6, cfg.hidden))
    first = mla.forward(x0, w, cfg)
    cache = (first["c_hat"], first["k_pe"])
    rows = np.array([0, 3, 5])
    a = mla.forward(x1, w, cfg, cache=cache, rows=rows)
    b = mla.forward(x1, w, cfg, cache=cache, rows=rows, absorbed=True)
    assert np.allclose(a["y"], b["y"], rtol=0, atol=1e-12)
    assert np.allclose(a["o"], b["o"], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ P9, P11
def test_prefill_equals_prefill_then_decode():
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=17)
    x = np.random.default_rng(18).standard_normal((9, cfg.hidden))
    full = mla.forward(x, w, cfg)
    first = mla.forward(x[:8], w, cfg)
    step = mla.forward(x[8:], w, cfg, cache=(first["c_hat"], first["k_pe"]))
    assert np.allclose(step["y"][0], full["y"][8], rtol=0, atol=1e-12)
    assert np.allclose(first["y"], full["y"][:8], rtol=0, atol=1e-12)


def test_causality_later_tokens_do_not_change_earlier_outputs():
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=19)
    rng = np.random.default_rng(20)
    x = rng.standard_normal((8, cfg.hidden))
    x2 = x.copy()
    x2[5:] = rng.standard_normal((3, cfg.hidden))
    a = mla.forward(x, w, cfg)["y"]
    b = mla.forward(x2, w, cfg)["y"]
    assert np.array_equal(a[:5], b[:5])
    assert not np.allclose(a[5:], b[5:])


def test_rows_subset_matches_full():
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=21)
    x = np.random.default_rng(22).standard_normal((10, cfg.hidden))
    full = mla.forward(x, w, cfg)
    sub = mla.forward(x, w, cfg, rows=np.array([0, 4, 9]))
    assert np.allclose(sub["y"], full["y"][[0, 4, 9]], rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------ P13, P14 FP8
def test_e4m3_decode_matches_torch_for_all_codes():
    import torch

    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8.e4m3_value(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_with_saturation():
    import torch

    rng = np.random.default_rng(23)
    vals = fp8.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties
    x = np.concatenate([
        rng.standard_normal(200000) * 50, rng.standard_normal(20000) * 1e-3, mids, -mids, vals, -vals,
        np.array([448.0, 449.0, 464.0, 1000.0, -500.0, 0.0, 1e-30]),
    ]).astype(np.float32)
    mine = fp8.e4m3_encode(x)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # compare values (a negative number rounding to zero may give +0 or -0)
    assert np.array_equal(fp8.e4m3_value(mine), fp8.e4m3_value(ref))
    assert not np.any((mine & 0x7F) == 0x7F)


def test_activation_quantiser_worked_cases():
    # a group whose amax is 448 * 2^-5 gets scale exactly 2^-5; exact e4m3 multiples round-trip
    g = np.zeros((1, 128))
    g[0, 0] = 448 * 2.0 ** -5
    g[0, 1] = -1.5 * 2.0 ** -5
    g[0, 2] = 0.65625 * 2.0 ** -5  # halfway between 0.625 (m=2) and 0.6875 (m=3): tie -> even m
    codes, s = fp8.quantize_1x128(g)
    assert s[0, 0] == np.float32(2.0 ** -5)
    dq = fp8.dequant_1x128(codes, s)
    assert dq[0, 0] == g[0, 0] and dq[0, 1] == g[0, 1]
    assert fp8.e4m3_value(codes[0, 2:3])[0] == 0.625
    # zero group -> scale 1, codes 0; groups are independent
    z = np.zeros((2, 256))
    z[1, 128:] = np.linspace(-3, 3, 128)
    c2, s2 = fp8.quantize_1x128(z)
    assert s2[0, 0] == 1.0 and s2[0, 1] == 1.0 and s2[1, 0] == 1.0 and np.all(c2[0] == 0)
    assert s2[1, 1] == np.float32(np.float32(3.0) / np.float32(448.0))
    # the largest element quantises to +-448 (possibly by saturation)
    assert np.max(np.abs(fp8.e4m3_value(c2[1, 128:]))) == 448.0
    # per-token groups: quantising rows one by one equals quantising the matrix
    m = np.random.default_rng(24).standard_normal((5, 384))
    cm, sm = fp8.quantize_1x128(m)
    for r in range(5):
        cr, sr = fp8.quantize_1x128(m[r:r + 1])
        assert np.array_equal(cr[0], cm[r]) and np.array_equal(sr[0], sm[r])


def test_weight_dequant_blocks_and_ragged_rows():
    rng = np.random.default_rng(25)
    codes = rng.integers(0, 0x7E, size=(576, 256)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, size=(5, 2)).astype(np.float32)
    w = fp8.dequant_weight(codes, s)
    v = fp8.e4m3_value(codes)
    assert w[0, 0] == v[0, 0] * float(s[0, 0])
    assert w[575, 255] == v[575, 255] * float(s[4, 1])  # ragged last block row (rows 512..575)
    assert w[511, 128] == v[511, 128] * float(s[3, 1])
    # exact: a 4-bit significand times a 24-bit significand fits in float64
    assert np.array_equal(w / np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:576, :256], v)


def test_w8a8_forward_quantises_projection_inputs():
    """W8A8 mode differs from plain mode only through the quantiser; with inputs that are
    already exact e4m3 multiples of a power-of-two group scale the quantiser is the identity
    on x, so q_a/kv_a outputs agree exactly."""
    cfg = mla.Config(hidden=128, q_lora=128, kv_lora=128, heads=2, nope=64, rope=64, v=64)
    w = tiny_weights(cfg, seed=26)
    x = np.zeros((1, 128))
    x[0, :4] = [448.0, -2.0, 1.0, 0.5]
    a = mla.latent_path(x, w, np.array([0]), cfg, w8a8=False)
    b = mla.latent_path(x, w, np.array([0]), cfg, w8a8=True)
    assert np.array_equal(a["ckv"], b["ckv"])
    # c_hat in W8A8 is the quantise-dequantise image of the RMSNorm output
    assert np.array_equal(b["c_hat"], fp8.fake_quant_1x128(a["c_hat"]))


# ------------------------------------------------------------------------ decoder-block wrapper
def test_round_bf16_matches_torch_on_float32_values():
    """The oracle's bf16 rounding against torch's float32 -> bfloat16 cast (round to nearest even)
    on float32 values, ties included (float64 inputs would see torch round twice)."""
    import torch

    rng = np.random.default_rng(21)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    # exact halfway cases over the normal range (the oracle rounds normal values only)
    ties = (np.arange(0x0080, 0x7F00, 7, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, 1.0, -2.5])]).astype(np.float64)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mla.round_bf16(v), want)


def test_block_residual_when_o_proj_vanishes():
    """W_o = 0: the attention adds nothing, so the block returns its (bf16) input exactly."""
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=31, zero=("o",))
    rng = np.random.default_rng(32)
    x = mla.round_bf16(rng.standard_normal((5, cfg.hidden)))
    g = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    out = mla.block_attention(x, w, g, cfg)
    assert np.array_equal(out["h"], x)


@pytest.mark.parametrize("c", [4.0, 0.25])
def test_block_input_norm_scale_invariance(c):
    """With eps = 0 the RMSNorm output does not depend on the input's scale (and a power-of-two
    scale leaves every bf16 rounding unchanged), so the layer output y is the same for x and c x,
    and h(c x) is c x + y rounded to bf16: a bf16 value within half a bf16 unit of c x + y. Fails
    if the norm were skipped, applied to the residual, or its output added instead of x."""
    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6, eps=0.0)
    w = tiny_weights(cfg, seed=33)
    rng = np.random.default_rng(34)
    x = rng.standard_normal((4, cfg.hidden))
    g = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    a = mla.block_attention(x, w, g, cfg)
    b = mla.block_attention(c * x, w, g, cfg)
    assert np.max(np.abs(a["y"] - b["y"])) <= 1e-12 * np.max(np.abs(a["y"]))
    want = c * x + a["y"]
    half_unit = np.ldexp(1.0, np.frexp(want)[1] - 9)  # half of 2^(e-8), the bf16 spacing at want
    assert np.all(np.abs(b["h"] - want) <= half_unit)
    bits = b["h"].astype(np.float32).view(np.uint32)
    assert np.all(b["h"].astype(np.float32) == b["h"]) and np.all(bits & 0xFFFF == 0)


def test_block_output_is_bf16_like_torch():
    """The block output h = x + y is a bf16 tensor (the model dtype): the oracle's rounding of the
    exact sum of a bf16 x and a float32-representable y equals torch's float32 add of the two
    followed by one cast to bfloat16, wherever that float32 sum is exact (most elements here;
    elsewhere torch would round twice)."""
    import torch

    cfg = mla.Config(hidden=64, q_lora=32, kv_lora=16, heads=4, nope=8, rope=8, v=6)
    w = tiny_weights(cfg, seed=37)
    rng = np.random.default_rng(38)
    x = mla.round_bf16(4.0 * rng.standard_normal((6, cfg.hidden)))
    g = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    out = mla.block_attention(x, w, g, cfg)
    y32 = out["y"].astype(np.float32)
    # the oracle's h from the float32 image of y (so that torch sees the same summands)
    want = mla.round_bf16(x + y32.astype(np.float64))
    s32 = torch.from_numpy(x.astype(np.float32)) + torch.from_numpy(y32)
    exact_sum = s32.double().numpy() == x + y32.astype(np.float64)
    assert exact_sum.mean() > 0.5
    assert np.array_equal(s32.to(torch.bfloat16).double().numpy()[exact_sum], want[exact_sum])
    # and the oracle's own h is the rounding of the unrounded sum, within half a unit of it
    exact = x + out["y"]
    assert np.all(np.abs(out["h"] - exact) <= np.ldexp(1.0, np.frexp(exact)[1] - 9))


@pytest.mark.parametrize("t_new,l0", [(3, 0), (1, 3)])
def test_block_brute_force_tiny(t_new, l0):
    """The block wrapper against the scalar-loop restatement (its own RMSNorm and bf16 rounding)."""
    cfg = TINY
    w = tiny_weights(cfg, seed=35)
    rng = np.random.default_rng(36 + t_new)
    g = 1.0 + 0.1 * rng.standard_normal(cfg.hidden)
    x_prev = rng.standard_normal((l0, cfg.hidden))
    x = rng.standard_normal((t_new, cfg.hidden))
    cache = None
    bcache = None
    if l0:
        cache = mla.kv_entries(mla.input_rmsnorm(x_prev, g, cfg.eps), w, 0, cfg)
        bcache = [(list(cache[0][i]), list(cache[1][i])) for i in range(l0)]
    out = mla.block_attention(x, w, g, cfg, cache=cache)
    dims = dict(q_lora=cfg.q_lora, kv_lora=cfg.kv_lora, heads=cfg.heads, nope=cfg.nope, rope=cfg.rope, v=cfg.v)
    hs, _ = brute.block(x.tolist(), to_lists(w), g.tolist(), dims, cfg.eps, cfg.theta, 1 / math.sqrt(cfg.qk), bcache)
    assert np.allclose(out["h"], np.array(hs), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------ W8A8 wiring, brute force
W8 = mla.Config(hidden=256, q_lora=128, kv_lora=128, heads=2, nope=64, rope=64, v=64)


def _w8_weights(seed):
    w = tiny_weights(W8, seed=seed)
    return {k: (v if k.endswith("norm") else 0.1 * v) for k, v in w.items()}


def _w8_case(t_new, l0, seed):
    w = _w8_weights(seed)
    rng = np.random.default_rng(seed + 1)
    x_prev = rng.standard_normal((l0, W8.hidden))
    x = rng.standard_normal((t_new, W8.hidden))
    cache = mla.kv_entries(x_prev, w, 0, W8, w8a8=True) if l0 else None
    bcache = [(list(cache[0][i]), list(cache[1][i])) for i in range(l0)] if l0 else None
    dims = dict(q_lora=W8.q_lora, kv_lora=W8.kv_lora, heads=W8.heads, nope=W8.nope, rope=W8.rope, v=W8.v)

    def run_brute(points):
        return brute.forward(x.tolist(), to_lists(w), dims, W8.eps, W8.theta, W8.sigma, bcache, w8a8=points)

    return mla.forward(x, w, W8, cache=cache, w8a8=True), run_brute


@pytest.mark.parametrize("t_new,l0", [(3, 0), (1, 3)])
def test_w8a8_forward_against_scalar_brute_force(t_new, l0):
    """The W8A8 layer (every projection input quantised: x into q_a and kv_a, q_hat into q_b,
    c_hat into kv_b, o into o_proj) against the scalar restatement with its own quantiser, at
    dimensions that are multiples of the 128-feature group. Prefill (T = 3) and a decode step
    onto a W8A8 cache."""
    out, run_brute = _w8_case(t_new, l0, seed=40 + l0)
    ys, ents = run_brute(brute.W8A8_POINTS)
    tol = 1e-12 * max(1.0, float(np.max(np.abs(out["y"]))))
    assert np.allclose(out["y"], np.array(ys), rtol=0, atol=tol)
    assert np.allclose(out["c_hat"], np.array([e[0] for e in ents]), rtol=0, atol=1e-12)
    assert np.allclose(out["k_pe"], np.array([e[1] for e in ents]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dropped", brute.W8A8_POINTS)
def test_w8a8_each_quantised_input_is_observable(dropped):
    """Leaving any one of the four quantisation points out of the brute force moves the output
    far beyond rounding: a wiring mistake at that point in the oracle would fail the test above."""
    out, run_brute = _w8_case(2, 2, seed=44)
    ys, _ = run_brute(tuple(p for p in brute.W8A8_POINTS if p != dropped))
    assert np.max(np.abs(out["y"] - np.array(ys))) > 1e-6 * np.max(np.abs(out["y"]))


def test_scalar_quantiser_matches_worked_e4m3_values():
    """The brute force's scalar e4m3 rounding: exact codes, a tie to the even significand,
    the subnormal spacing 2^-9, saturation at 448."""
    assert brute._e4m3(448.0) == 448.0 and brute._e4m3(1000.0) == 448.0 and brute._e4m3(-460.0) == -448.0
    assert brute._e4m3(0.65625) == 0.625            # halfway between 0.625 (m=2) and 0.6875 (m=3)
    assert brute._e4m3(0.71875) == 0.75             # halfway between 0.6875 (m=3) and 0.75 (m=4)
    assert brute._e4m3(3 * 2.0 ** -10) == 2.0 ** -8  # 1.5 subnormal steps: tie to the even step 2
    assert brute._e4m3(2.0 ** -9) == 2.0 ** -9 and brute._e4m3(2.0 ** -11) == 0.0
    assert brute._e4m3(240.0) == 240.0 and brute._e4m3(250.0) == 256.0


@pytest.mark.parametrize("w8a8", [False, True])
def test_kv_entries_chunks_equal_one_pass(w8a8):
    """Cache filling in chunks (here 3 tokens, so 7 tokens cross two chunk boundaries) gives the
    entries the scalar brute force computes for positions 0..6 in one pass."""
    w = _w8_weights(46)
    x = np.random.default_rng(47).standard_normal((7, W8.hidden))
    c, k = mla.kv_entries(x, w, 0, W8, w8a8=w8a8, chunk=3)
    dims = dict(q_lora=W8.q_lora, kv_lora=W8.kv_lora, heads=W8.heads, nope=W8.nope, rope=W8.rope, v=W8.v)
    _, ents = brute.forward(x.tolist(), to_lists(w), dims, W8.eps, W8.theta, W8.sigma,
                            w8a8=brute.W8A8_POINTS if w8a8 else ())
    assert np.allclose(c, np.array([e[0] for e in ents]), rtol=0, atol=1e-12)
    assert np.allclose(k, np.array([e[1] for e in ents]), rtol=0, atol=1e-12)
    # a later start position: chunks continue the positions
    c5, k5 = mla.kv_entries(x, w, 5, W8, w8a8=w8a8, chunk=3)
    lat = mla.latent_path(x, w, 5 + np.arange(7), W8, w8a8=w8a8)
    assert np.allclose(c5, lat["c_hat"], rtol=0, atol=1e-12) and np.allclose(k5, lat["k_pe"], rtol=0, atol=1e-12)
