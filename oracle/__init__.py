"""Float64 CPU oracle for one Multi-head Latent Attention layer (Kimi-K2 dimensions).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link anything in
this package: only the tests, the smoke check and the bench's CPU-baseline leg use it. It is
a plain, slow, obviously correct restatement of what the reference pages define, written in
numpy float64 (library matmul as the only primitive), and it shares no code with the HIP
path. Inputs arrive as float64 arrays (bf16 or e4m3 values upcast exactly).

Modules:
  mla   -- the layer: projections, RMSNorm, RoPE, latent cache entries, rebuilt keys and
           values, causal softmax attention, output projection; also the absorbed
           (latent-space) form used only as a cross-check.
  fp8   -- OCP E4M3FN decode/encode, the 128x128 block weight dequantiser and the dynamic
           1x128 activation quantiser.
  brute -- a pure-Python scalar-loop restatement for tiny dimensions (independent pin).

Readings taken where the pages are silent (each also listed in the design notes):
  * query path = q_b(RMSNorm_q(q_a(x))), per head [128 content | 64 rotary];
  * softmax scale = 1/sqrt(192) (the scale is used but never defined on the pages);
  * RoPE pairs features (2i, 2i+1) of the 64 rotary features, frequency theta^(-2i/64),
    angle = absolute position * frequency, no YaRN correction;
  * causal mask: key position j visible to query position p iff j <= p;
  * the cache holds positions 0..L-1 contiguously; this call's entries are appended before
    attention, so a decode step sees L+1 positions including its own;
  * FP8 activations: per token, per aligned group of 128 inputs, s = fl32(amax/448),
    code = RNE-e4m3(saturate(fl32(a/s))), amax == 0 -> s = 1.

Parity unpinned (fixed by the readings above, not by any value the pages print): the RoPE
pairing convention, the softmax scale, the absence of YaRN, and the FP8 activation
quantiser's granularity and scale formula.
"""
from . import fp8, mla  # noqa: F401
