"""Float64 oracle of one MLA layer. TEST INFRASTRUCTURE ONLY (see the package docstring).

Every array is float64. Weights are [out, in] ("Key content up-projection" page, Parameters:
the module holds its weight output by input), so a projection is y = x @ W.T.

Sources, by page and section:
  * module inventory and widths: "Key-value latent" page, mla-init excerpt;
  * kv path (split 512 | 64, latent RMSNorm, kv_b, per-head split 128 | 128): same page,
    mla-kv excerpt;
  * RMSNorm: same page, rmsnorm excerpt;
  * query/key assembly, cache update, scaled scores, size checks, mask, float32 softmax,
    dropout, P.V: "Key content up-projection" page, code excerpt (mla-prefill);
  * head flattening and o_proj: dense-block attention page (prefill), mla-output excerpt;
  * W_UK = output features 0..127 of each head's 256 in kv_b: "Key content up-projection"
    page, Explanation;
  * cache returns every position so far (1,001 at p = 1000): "KV cache" page, state card.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import fp8 as _fp8


@dataclass(frozen=True)
class Config:
    """Layer hyper-parameters (Kimi-K2 values from the config excerpt on the "KV cache" page)."""

    hidden: int = 7168
    q_lora: int = 1536
    kv_lora: int = 512
    heads: int = 64
    nope: int = 128
    rope: int = 64
    v: int = 128
    eps: float = 1e-6          # rms_norm_eps (also the RMSNorm default in the rmsnorm excerpt)
    theta: float = 50000.0     # rope_theta
    scale: float | None = None  # softmax scale; None -> 1/sqrt(nope + rope) [x YaRN factor^2]
    # YaRN RoPE (rope_scaling in the same config excerpt); rope_factor <= 1 means plain RoPE
    rope_factor: float = 1.0
    rope_orig_max: int = 4096   # original_max_position_embeddings
    beta_fast: float = 1.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 1.0

    @property
    def qk(self) -> int:
        return self.nope + self.rope

    @property
    def yarn(self) -> bool:
        return self.rope_factor > 1.0

    @property
    def sigma(self) -> float:
        if self.scale is not None:
            return self.scale
        base = 1.0 / np.sqrt(float(self.qk))
        if self.yarn:
            f = yarn_attention_factor(self.rope_factor, self.mscale_all_dim)
            base *= f * f
        return base

    @property
    def rope_gain(self) -> float:
        """Multiplier on the rotary cos/sin (1 without YaRN)."""
        if not self.yarn:
            return 1.0
        return yarn_attention_factor(self.rope_factor, self.mscale) / yarn_attention_factor(self.rope_factor, self.mscale_all_dim)


KIMI_K2 = Config()
# The released configuration's rope_scaling (config excerpt on the "KV cache" page): YaRN with
# factor 32 over an original 4,096 positions, beta_fast = beta_slow = 1, mscale = mscale_all_dim = 1.
KIMI_K2_YARN = Config(rope_factor=32.0)


def yarn_attention_factor(s: float, m: float) -> float:
    """YaRN's attention temperature factor sqrt(1/t) = 0.1 m ln(s) + 1 (YaRN paper, Peng et al.
    2023, section 3.4, with m the config's mscale coefficient); 1 when s <= 1."""
    return 1.0 if s <= 1.0 else 0.1 * m * np.log(s) + 1.0


def yarn_frequencies(rope: int, theta: float, s: float, orig_max: int, beta_fast: float,
                     beta_slow: float) -> np.ndarray:
    """Per-pair rotary frequencies under YaRN's "NTK-by-parts" rule (YaRN paper, section 3.2).

    Pair i has base frequency theta_i = theta^(-2i/rope), wavelength 2 pi / theta_i and
    r_i = orig_max / wavelength_i turns over the original context. A pair that turns often
    (r >= beta_fast) keeps theta_i; one that turns less than beta_slow times is interpolated to
    theta_i / s; in between the two are blended linearly in r. With beta_fast == beta_slow (the
    released configuration) the blend is a step at r = beta_fast.
    """
    i = np.arange(rope // 2, dtype=np.float64)
    freq = theta ** (-2.0 * i / rope)
    r = orig_max * freq / (2.0 * np.pi)
    if beta_fast > beta_slow:
        gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    else:
        gamma = (r >= beta_fast).astype(np.float64)
    return (1.0 - gamma) * freq / s + gamma * freq


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """nn.Linear without bias (attention_bias is false): y = x W^T."""
    return x @ w.T


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis ("Key-value latent" page, rmsnorm excerpt).

    y = g * x / sqrt(mean(x^2) + eps). The excerpt computes in float32 and casts back to the
    input dtype before the gain; here nothing is rounded (float64 throughout).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def rope_cos_sin(pos: np.ndarray, rope: int, theta: float, cfg: Config | None = None) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin of the rotary angles, [len(pos), rope/2] ("32 pairs" input on the dense-block
    attention page). Pair i has frequency theta^(-2i/rope); the angle is position * frequency.
    With a YaRN config (cfg.rope_factor > 1) the frequencies are yarn_frequencies() and cos/sin
    carry cfg.rope_gain.
    """
    if cfg is not None and cfg.yarn:
        freq = yarn_frequencies(rope, theta, cfg.rope_factor, cfg.rope_orig_max, cfg.beta_fast, cfg.beta_slow)
        gain = cfg.rope_gain
    else:
        i = np.arange(rope // 2, dtype=np.float64)
        freq = theta ** (-2.0 * i / rope)
        gain = 1.0
    ang = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]
    return gain * np.cos(ang), gain * np.sin(ang)


def rope_rotate(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate features (2i, 2i+1) by the pair-i angle: (a, b) -> (a c - b s, a s + b c).

    v is [T, ..., rope]; cos/sin are [T, rope/2] and broadcast over the middle axes.
    """
    shape = (cos.shape[0],) + (1,) * (v.ndim - 2) + (cos.shape[1],)
    c = cos.reshape(shape)
    s = sin.reshape(shape)
    a = v[..., 0::2]
    b = v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _act(a: np.ndarray, w8a8: bool) -> np.ndarray:
    """Projection input: unchanged, or passed through the dynamic FP8 quantiser (W8A8)."""
    return _fp8.fake_quant_1x128(a) if w8a8 else a


def query_path(x: np.ndarray, w: dict, pos: np.ndarray, cfg: Config = KIMI_K2, w8a8: bool = False) -> dict:
    """q_a -> q RMSNorm -> q_b, split per head into content (nope) and rotary (pe), rotate pe.

    The query forward is not excerpted on the pages; this is the reading that the module list
    (mla-init excerpt) and the assembly order (mla-prefill excerpt) support.
    """
    cq = linear(_act(x, w8a8), w["q_a"])
    q_hat = rmsnorm(cq, w["q_a_norm"], cfg.eps)
    q = linear(_act(q_hat, w8a8), w["q_b"]).reshape(x.shape[0], cfg.heads, cfg.qk)
    cos, sin = rope_cos_sin(pos, cfg.rope, cfg.theta, cfg)
    return {
        "cq": cq,
        "q_hat": q_hat,
        "q_nope": q[..., : cfg.nope],
        "q_pe": rope_rotate(q[..., cfg.nope:], cos, sin),
    }


def latent_path(x: np.ndarray, w: dict, pos: np.ndarray, cfg: Config = KIMI_K2, w8a8: bool = False) -> dict:
    """kv_a_proj_with_mqa -> split [512 latent | 64 shared rotary key] -> latent RMSNorm; rotate
    the shared key ("Key-value latent" page, mla-kv excerpt).

    Returns the latent cache entry of each token: c_hat (the RMSNorm output, the input of
    kv_b) and k_pe (rotated). In W8A8 mode c_hat is the quantise-dequantise image of the
    RMSNorm output, because that is what kv_b consumes.
    """
    ckv = linear(_act(x, w8a8), w["kv_a"])
    c = ckv[:, : cfg.kv_lora]
    k_pe = ckv[:, cfg.kv_lora:]
    c_hat = rmsnorm(c, w["kv_a_norm"], cfg.eps)
    if w8a8:
        c_hat = _fp8.fake_quant_1x128(c_hat)
    cos, sin = rope_cos_sin(pos, cfg.rope, cfg.theta, cfg)
    return {"ckv": ckv, "c_hat": c_hat, "k_pe": rope_rotate(k_pe, cos, sin)}


def rebuild_kv(c_hat: np.ndarray, k_pe: np.ndarray, w_kvb: np.ndarray, cfg: Config = KIMI_K2):
    """Rebuilt keys and values from latent entries ("Key-value latent" page, mla-kv; "Key content
    up-projection" page, code excerpt): kv = c_hat W_kvb^T viewed [L, heads, 128 + 128];
    K = [k_nope | k_pe shared by every head] ([L, heads, 192]); V = [L, heads, 128].
    """
    n = c_hat.shape[0]
    kv = linear(c_hat, w_kvb).reshape(n, cfg.heads, cfg.nope + cfg.v)
    k = np.empty((n, cfg.heads, cfg.qk))
    k[..., : cfg.nope] = kv[..., : cfg.nope]
    k[..., cfg.nope:] = k_pe[:, None, :]
    return k, kv[..., cfg.nope:]


def attend(q_nope: np.ndarray, q_pe: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
           sigma: float) -> np.ndarray:
    """Causal scaled-dot-product attention, per query and head.

    q_* are [Tq, heads, *]; k is [L, heads, 192] and v [L, heads, 128], row j holding key
    position j. Query t at position q_pos[t] sees keys 0..q_pos[t] (the causal mask: masked
    weights are exactly zero). Scores are sigma * q.k over 192 features; softmax is taken with
    the maximum subtracted; dropout p = 0 is the identity. Returns o [Tq, heads, 128].
    """
    q = np.concatenate([q_nope, q_pe], axis=-1)
    tq, heads, _ = q.shape
    o = np.empty((tq, heads, v.shape[-1]))
    for t in range(tq):
        n = int(q_pos[t]) + 1
        s = np.einsum("hd,jhd->hj", q[t], k[:n]) * sigma
        s = s - s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a = a / a.sum(axis=1, keepdims=True)
        o[t] = np.einsum("hj,jhd->hd", a, v[:n])
    return o


def forward(x: np.ndarray, w: dict, cfg: Config = KIMI_K2, cache: tuple | None = None,
            rows: np.ndarray | None = None, w8a8: bool = False, absorbed: bool = False) -> dict:
    """One MLA call for ONE sequence: prefill (T tokens) or decode (T = 1) on a latent cache.

    x        [T, hidden] float64, this call's tokens.
    w        float64 weights keyed q_a, q_a_norm, q_b, kv_a, kv_a_norm, kv_b, o (FP8 weights are
             passed already dequantised).
    cache    (c_hat [L0, kv_lora], k_pe [L0, rope]) entries of positions 0..L0-1, or None.
    rows     indices into this call's tokens whose outputs are wanted (default: all).
    w8a8     pass every projection input through the dynamic FP8 activation quantiser.
    absorbed attend in the 512-feature latent space (attend_absorbed) instead of rebuilding
             per-head keys and values for every cached position: the same values (pinned
             against the rebuilt form), at a cost that stays small for tens of thousands of
             cached positions.

    Token t sits at position L0 + t. All T entries are appended to the cache before the
    scores are formed, so the keys cover positions 0..L0+T-1 and the causal mask limits each
    query to its own position.

    Returns y [len(rows), hidden], o [len(rows), heads*v] (the o_proj input), the new cache
    entries (c_hat, k_pe) of all T tokens, and the query intermediates of `rows`.
    """
    t_new = x.shape[0]
    l0 = 0 if cache is None else cache[0].shape[0]
    pos = l0 + np.arange(t_new)
    rows = np.arange(t_new) if rows is None else np.asarray(rows)

    lat = latent_path(x, w, pos, cfg, w8a8)
    if cache is None:
        c_all, kpe_all = lat["c_hat"], lat["k_pe"]
    else:
        c_all = np.concatenate([cache[0], lat["c_hat"]], axis=0)
        kpe_all = np.concatenate([cache[1], lat["k_pe"]], axis=0)
    n_keys = l0 + int(rows.max()) + 1 if rows.size else 0
    qp = query_path(x[rows], w, pos[rows], cfg, w8a8)
    if absorbed:
        o = attend_absorbed(qp["q_nope"], qp["q_pe"], c_all[:n_keys], kpe_all[:n_keys], w["kv_b"], pos[rows], cfg)
    else:
        k, v = rebuild_kv(c_all[:n_keys], kpe_all[:n_keys], w["kv_b"], cfg)
        o = attend(qp["q_nope"], qp["q_pe"], k, v, pos[rows], cfg.sigma)
    o_flat = o.reshape(len(rows), cfg.heads * cfg.v)  # index h*128 + d
    y = linear(_act(o_flat, w8a8), w["o"])
    return {"y": y, "o": o_flat, "c_hat": lat["c_hat"], "k_pe": lat["k_pe"], "ckv": lat["ckv"], **qp}


def kv_entries(x: np.ndarray, w: dict, pos0: int = 0, cfg: Config = KIMI_K2, w8a8: bool = False,
               chunk: int = 4096) -> tuple[np.ndarray, np.ndarray]:
    """Latent cache entries (c_hat, k_pe) for tokens at positions pos0, pos0+1, ...

    An entry depends only on its own token and position, so this is the kv part of `forward`
    applied in chunks (used to fill long caches without running attention).
    """
    cs, ks = [], []
    for s in range(0, x.shape[0], chunk):
        xs = x[s:s + chunk]
        lat = latent_path(xs, w, pos0 + s + np.arange(xs.shape[0]), cfg, w8a8)
        cs.append(lat["c_hat"])
        ks.append(lat["k_pe"])
    return np.concatenate(cs), np.concatenate(ks)


# ----------------------------------------------------------------------------------------------
# attention half of a decoder block: input RMSNorm, the layer, residual addition
# ----------------------------------------------------------------------------------------------
def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (8 significant bits), in float64.

    frexp gives v = m * 2^e with 0.5 <= |m| < 1; the significand m * 2^8 is rounded to an
    integer (numpy rounds halves to even) and scaled back. Values stay in the normal range here.
    """
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def input_rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """The block's input RMSNorm with the dtype flow of the rmsnorm excerpt ("Attention input"
    page): the normalised activation is cast back to the input dtype (bf16) before the gain, and
    the product of the bf16 gain with it is again a bf16 tensor -- the layer's bf16 input. So
    y = bf16(g * bf16(x / sqrt(mean(x^2) + eps))), with the mean and root exact in float64.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return round_bf16(g * round_bf16(x / np.sqrt(ms + eps)))


def block_attention(x: np.ndarray, w: dict, g_in: np.ndarray, cfg: Config = KIMI_K2, cache: tuple | None = None,
                    rows: np.ndarray | None = None, w8a8: bool = False, absorbed: bool = False) -> dict:
    """Attention half of a decoder block ("Attention input" page, block excerpt): the residual
    is the block input, the layer sees its input RMSNorm (gain g_in over the hidden features,
    eps = rms_norm_eps), and the layer output is added to the residual: h = x + MLA(norm(x)).

    The block's output is the model's hidden state, a tensor of the model dtype (bf16: the
    config excerpt's torch_dtype): h is the bf16 rounding of the exact sum x + y, where the
    layer output y itself stays unrounded (float64) as everywhere in the oracle. A stack of
    blocks therefore passes bf16 hidden states from one block to the next, as the model does.

    Same arguments as `forward`; returns h [len(rows), hidden], the normalised input xn and
    everything `forward` returns for it (y is the unrounded layer output).
    """
    xn = input_rmsnorm(x, g_in, cfg.eps)
    out = forward(xn, w, cfg, cache=cache, rows=rows, w8a8=w8a8, absorbed=absorbed)
    r = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    return {"h": round_bf16(x[r] + out["y"]), "xn": xn, **out}


# ----------------------------------------------------------------------------------------------
# absorbed (latent-space) form -- a cross-check of the algebra, not the definition
# ----------------------------------------------------------------------------------------------
def attend_absorbed(q_nope: np.ndarray, q_pe: np.ndarray, c_hat: np.ndarray, k_pe: np.ndarray,
                    w_kvb: np.ndarray, q_pos: np.ndarray, cfg: Config = KIMI_K2) -> np.ndarray:
    """Same result as rebuild_kv + attend, computed in the 512-feature latent space.

    With W_UK,h = rows h*256 .. h*256+127 of kv_b and W_UV,h = rows h*256+128 .. h*256+255
    ("Key content up-projection" page, Explanation): q_nope.(W_UK c) = (W_UK^T q_nope).c and
    sum_j a_j W_UV c_j = W_UV sum_j a_j c_j.
    """
    wk = w_kvb.reshape(cfg.heads, cfg.nope + cfg.v, cfg.kv_lora)
    w_uk, w_uv = wk[:, : cfg.nope, :], wk[:, cfg.nope:, :]
    q_lat = np.einsum("thd,hdc->thc", q_nope, w_uk)  # [Tq, heads, kv_lora]
    tq = q_nope.shape[0]
    o = np.empty((tq, cfg.heads, cfg.v))
    for t in range(tq):
        n = int(q_pos[t]) + 1
        s = (q_lat[t] @ c_hat[:n].T + q_pe[t] @ k_pe[:n].T) * cfg.sigma
        s = s - s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a = a / a.sum(axis=1, keepdims=True)
        o_lat = a @ c_hat[:n]  # [heads, kv_lora]
        o[t] = np.einsum("hc,hdc->hd", o_lat, w_uv)
    return o


# ----------------------------------------------------------------------------------------------
# sizes printed on the pages
# ----------------------------------------------------------------------------------------------
def weight_shapes(cfg: Config = KIMI_K2) -> dict[str, tuple[int, ...]]:
    """Parameter tensor shapes implied by the mla-init excerpt ("Key-value latent" page)."""
    return {
        "q_a": (cfg.q_lora, cfg.hidden),
        "q_a_norm": (cfg.q_lora,),
        "q_b": (cfg.heads * cfg.qk, cfg.q_lora),
        "kv_a": (cfg.kv_lora + cfg.rope, cfg.hidden),
        "kv_a_norm": (cfg.kv_lora,),
        "kv_b": (cfg.heads * (cfg.qk - cfg.rope + cfg.v), cfg.kv_lora),
        "o": (cfg.hidden, cfg.heads * cfg.v),
    }


def cache_bytes_per_position(cfg: Config = KIMI_K2, elem_bytes: int = 2) -> dict[str, int]:
    """Bytes one position occupies per layer: rebuilt keys+values vs latent + rotary key."""
    return {
        "rebuilt": cfg.heads * (cfg.qk + cfg.v) * elem_bytes,
        "latent": (cfg.kv_lora + cfg.rope) * elem_bytes,
        "flash_padded": cfg.heads * (cfg.qk + cfg.qk) * elem_bytes,
    }
