"""Pure-Python scalar-loop MLA layer for tiny dimensions. TEST INFRASTRUCTURE ONLY.

An independent restatement of the same equations as `oracle.mla` (no numpy, no shared code),
used to pin the vectorised oracle by brute force on tiny shapes (hidden 8, ranks 4-6, 2 heads,
head widths 2-4, a handful of tokens). Every loop follows one equation of the pages:

  "Key-value latent" page, mla-init / mla-kv / rmsnorm excerpts;
  "Key content up-projection" page, code excerpt (assembly, scores, mask, softmax, P.V);
  dense-block attention page, mla-output excerpt (flatten heads, o_proj);
  "Attention input" page, block and rmsnorm excerpts (input RMSNorm in bf16, residual add);
  "Key-value latent" page, linear excerpt (FP8 e4m3 weights, "dynamic" activations): in W8A8
  mode every projection input passes through a scalar restatement of the dynamic quantiser
  (per token and aligned group of 128 features, scale fl32(amax / 448), RNE e4m3 codes with
  saturation), written from the E4M3FN bit layout with IEEE single rounding via `struct`.
"""
from __future__ import annotations

import math
import struct

# projection inputs that the W8A8 mode quantises (a test may drop one to show it matters)
W8A8_POINTS = ("x", "q_hat", "c_hat", "o")


def _f32(v):
    """Round a Python float to IEEE single precision (round to nearest even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _e4m3(t):
    """Nearest E4M3FN value of t (ties to the even significand), saturating at +-448.

    E4M3FN: 3 stored significand bits; normal binades 2^-6 .. 2^8 (exponent field 1..15,
    bias 7, largest finite 1.75 * 2^8 = 448); below 2^-6 the spacing is 2^-9 (subnormals).
    """
    a = min(abs(t), 448.0)
    if a == 0.0:
        return 0.0
    m, e = math.frexp(a)            # a = m * 2^e, 0.5 <= m < 1, so the leading bit is 2^(e-1)
    step = 2.0 ** max(e - 4, -9)    # three bits after the leading one; subnormal spacing 2^-9
    q = a / step                    # exact: a power-of-two divisor
    r = math.floor(q)
    d = q - r
    if d > 0.5 or (d == 0.5 and r % 2 == 1):
        r += 1
    v = min(r * step, 448.0)
    return -v if t < 0 else v


def _quant(row):
    """Dynamic activation quantiser on one token's features: value seen by the projection."""
    out = []
    for g0 in range(0, len(row), 128):
        grp = [_f32(v) for v in row[g0:g0 + 128]]
        amax = max(abs(v) for v in grp)
        s = _f32(amax / 448.0) if amax > 0.0 else 1.0
        out.extend(_e4m3(_f32(v / s)) * s for v in grp)
    return out


def _matvec(w, x):
    """y[o] = sum_i w[o][i] * x[i]  (nn.Linear, [out, in] weight, no bias)."""
    return [sum(w[o][i] * x[i] for i in range(len(x))) for o in range(len(w))]


def _rms(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [g[i] * x[i] * r for i in range(len(x))]


def _rotate(v, p, theta):
    """Pairs (2i, 2i+1) rotated by angle p * theta^(-2i/len(v))."""
    out = list(v)
    n = len(v)
    for i in range(n // 2):
        ang = p * theta ** (-2.0 * i / n)
        c, s = math.cos(ang), math.sin(ang)
        a, b = v[2 * i], v[2 * i + 1]
        out[2 * i] = a * c - b * s
        out[2 * i + 1] = a * s + b * c
    return out


def forward(x, w, dims, eps, theta, sigma, cache_entries=None, w8a8=()):
    """x: list of T token vectors; w: dict of nested lists; dims: dict with keys
    q_lora, kv_lora, heads, nope, rope, v. cache_entries: list of (c_hat, k_pe) for positions
    0..L0-1. w8a8: the projection inputs (names in W8A8_POINTS) that pass through the dynamic
    FP8 quantiser first (all four for the W8A8 layer; the cached c_hat is then the quantised
    value kv_b consumes). Returns (y rows, new entries)."""
    heads, nope, rope, vd = dims["heads"], dims["nope"], dims["rope"], dims["v"]
    kv_lora = dims["kv_lora"]

    def act(point, v):
        return _quant(v) if point in w8a8 else v

    entries = list(cache_entries or [])
    l0 = len(entries)
    # keys and values: every token of this call is appended first
    for t, xt in enumerate(x):
        p = l0 + t
        ckv = _matvec(w["kv_a"], act("x", xt))
        c_hat = act("c_hat", _rms(ckv[:kv_lora], w["kv_a_norm"], eps))
        k_pe = _rotate(ckv[kv_lora:], p, theta)
        entries.append((c_hat, k_pe))
    keys, vals = [], []
    for c_hat, k_pe in entries:
        kv = _matvec(w["kv_b"], c_hat)
        kh, vh = [], []
        for h in range(heads):
            base = h * (nope + vd)
            kh.append(kv[base: base + nope] + list(k_pe))
            vh.append(kv[base + nope: base + nope + vd])
        keys.append(kh)
        vals.append(vh)
    ys = []
    for t, xt in enumerate(x):
        p = l0 + t
        q_hat = _rms(_matvec(w["q_a"], act("x", xt)), w["q_a_norm"], eps)
        q = _matvec(w["q_b"], act("q_hat", q_hat))
        o_flat = []
        for h in range(heads):
            base = h * (nope + rope)
            qh = q[base: base + nope] + _rotate(q[base + nope: base + nope + rope], p, theta)
            scores = []
            for j in range(p + 1):  # causal: keys at positions 0..p
                scores.append(sigma * sum(qh[d] * keys[j][h][d] for d in range(nope + rope)))
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            o_h = [sum(e[j] / z * vals[j][h][d] for j in range(p + 1)) for d in range(vd)]
            o_flat.extend(o_h)
        ys.append(_matvec(w["o"], act("o", o_flat)))
    return ys, entries[l0:]


def _bf16(v):
    """Nearest bfloat16 (8 significant bits, ties to even) of a Python float."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)          # v = m * 2**e, 0.5 <= |m| < 1
    q = m * 256.0
    r = math.floor(q)
    d = q - r
    if d > 0.5 or (d == 0.5 and r % 2 == 1):
        r += 1
    return math.ldexp(r, e - 8)


def block(x, w, g_in, dims, eps, theta, sigma, cache_entries=None):
    """h = bf16(x + layer(xn)) per token (the block output is a bf16 hidden state),
    xn = bf16(g_in * bf16(x / rms(x))). Returns (h rows, entries)."""
    xn = []
    for xt in x:
        r = 1.0 / math.sqrt(sum(v * v for v in xt) / len(xt) + eps)
        xn.append([_bf16(g_in[i] * _bf16(xt[i] * r)) for i in range(len(xt))])
    ys, ents = forward(xn, w, dims, eps, theta, sigma, cache_entries)
    return [[_bf16(x[t][i] + ys[t][i]) for i in range(len(x[t]))] for t in range(len(x))], ents
